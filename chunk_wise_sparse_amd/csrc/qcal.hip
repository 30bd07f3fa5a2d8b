// Q-Cal, the low-rank query calibration delta_q = W_up (W_down h)
// [HiLS Attention explainer (molayo1419.me), "Engineering details", Q-Cal item].
//
// Prefill splits it in two: this file computes the rank-r code t = W_down h for every token
// (an HBM-bound pass over h, on MFMA), and the selection kernel applies W_up per head inside
// its query tile.  Decode does both halves here for one token per sequence.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

// t[tok, a] = sum_D h[tok, D] * W_down[a, D], fp32.  One wave = TPW tiles of 16 tokens, four
// waves per workgroup; each W_down fragment is read once per wave and used for all TPW tiles.
// A operand = h rows (tokens), B operand = W_down rows (code index a), contraction over D.
// Each lane owns a 64-byte run of its row per 256-byte block: k index within the block is
// g * (4 * VL) + e, the same for A and B.  Rows past n_tok read the last token and are not
// stored.
template <typename T, int TPW>
__global__ __launch_bounds__(256) void prefill_qcal_code_kernel(const T* __restrict__ h,
                                                                const T* __restrict__ w_down,
                                                                float* __restrict__ t_out,
                                                                int n_tok, int D, int r) {
  constexpr int VL = 16 / sizeof(T);        // elements per 16-byte vector
  constexpr int KPL = Mfma<T>::KPL;
  constexpr int SUB = VL / KPL;             // MFMA steps per vector
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int tok0 = (blockIdx.x * 4 + wave) * 16 * TPW;
  const int nb = (r + 15) >> 4;             // code blocks of 16
  const T* hrow[TPW];
#pragma unroll
  for (int p = 0; p < TPW; ++p) hrow[p] = h + (size_t)min(tok0 + 16 * p + m, n_tok - 1) * D + g * 4 * VL;

  f32x4 acc[TPW][4];
#pragma unroll
  for (int p = 0; p < TPW; ++p)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[p][cb] = zero4();
  for (int base = 0; base < D; base += 16 * VL) {
    typedef T vecT __attribute__((ext_vector_type(VL)));
    vecT av[TPW][4];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int u = 0; u < 4; ++u) av[p][u] = *reinterpret_cast<const vecT*>(hrow[p] + base + u * VL);
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
          typename Mfma<T>::frag fb;
          if constexpr (KPL == 1) fb = bv[u][e];
          else {
#pragma unroll
            for (int z = 0; z < KPL; ++z) fb[z] = bv[u][e * KPL + z];
          }
#pragma unroll
          for (int p = 0; p < TPW; ++p) {
            typename Mfma<T>::frag fa;
            if constexpr (KPL == 1) fa = av[p][u][e];
            else {
#pragma unroll
              for (int z = 0; z < KPL; ++z) fa[z] = av[p][u][e * KPL + z];
            }
            acc[p][cb] = Mfma<T>::mma(fa, fb, acc[p][cb]);
          }
        }
      }
    }
  }
  // D[tok][a]: lane holds column a = 16cb + m, rows (tokens) 4g + rr of each tile.
#pragma unroll
  for (int p = 0; p < TPW; ++p)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (cb >= nb) break;
      const int a = cb * 16 + m;
      if (a < r) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int tok = tok0 + 16 * p + 4 * g + rr;
          if (tok < n_tok) t_out[(size_t)tok * r + a] = acc[p][cb][rr];
        }
      }
    }
}

template <typename T>
hipError_t launch_prefill_qcal_code(const T* h, const T* w_down, float* t_out, int n_tok, int D,
                                    int r, hipStream_t st) {
  constexpr int TPW = sizeof(T) == 2 ? 4 : 1;  // tokens per workgroup: 4 waves x 16 TPW
  const int per = 64 * TPW;
  hipLaunchKernelGGL((prefill_qcal_code_kernel<T, TPW>), dim3((n_tok + per - 1) / per), dim3(256), 0, st, h,
                     w_down, t_out, n_tok, D, r);
  return hipGetLastError();
}

template hipError_t launch_prefill_qcal_code<bf16>(const bf16*, const bf16*, float*, int, int, int, hipStream_t);
template hipError_t launch_prefill_qcal_code<float>(const float*, const float*, float*, int, int, int, hipStream_t);

}  // namespace hils

