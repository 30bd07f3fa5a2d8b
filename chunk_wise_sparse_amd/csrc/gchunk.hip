// HiLS prefill for chunk sizes C other than 64 (32 and 128), for the rows the MFMA kernels do not
// take: selection and attention for fp32, and for bf16 the selection of sequences that are not
// whole 64-query tiles (the chunk-major kernels attend afterwards).  The steps
// are the method's [HiLS-Attention model page, "Model Description"; HiLS Attention explainer
// (molayo1419.me), "Core idea" and "Engineering details"]: q~ = q + W_up t (Q-Cal), a score per
// causal chunk against its landmark key, the top-k chunks (ties to the smaller index; with the
// forced local chunk, the own chunk and the top k - 1 earlier ones), a softmax over their
// scores, and each chunk's causal softmax attention fused by those weights.
//
// The 64-key kernels tie their tiles to one 64-key chunk (a 64-query tile shares one candidate
// set, a chunk is one MFMA tile); this path has no such tie and no MFMA.  W waves own one query
// row (W = 1: each wave its own row, kGcRows rows per workgroup, for prefills with many rows;
// W = 4 for rows with more than 2048 chunks; W = 16 for launches of few
// rows).  The row's scores sit in LDS (up to 8192 chunks, sized to the launch's chunk count);
// the k-th largest is found by bisection over the order-preserving 32-bit keys with row-wide
// counts; the first wave then takes the keys above it and the earliest equal ones in chunk
// order.  The selected chunks are split over the row's waves: per chunk, lanes over keys form
// the scores and the causal softmax, then lanes over (key, 16-byte slice of d) accumulate the
// weighted values; every chunk's output is already normalised, so the waves' partial sums add.
// fp32 arithmetic throughout; q~ and the output are rounded once to the dtype.
#include "gchunk.h"
#include "hils_device.h"

namespace hils {

constexpr int kGcRows = 4;                     // rows per workgroup when W == 1
constexpr int kGcFewRows = 8192;               // launches of at most this many rows take W = 16
constexpr int kGcWideChunks = 2048;            // prefill rows with more chunks take W = 4

template <typename T, int D, int W>
__global__ __launch_bounds__(W == 1 ? 64 * kGcRows : 64 * W) void gchunk_kernel(const GcArgs a) {
  constexpr int SL = W == 1 ? kGcRows : 1;     // rows per workgroup
  constexpr int NW = W == 1 ? kGcRows : W;     // waves per workgroup
  constexpr int EPL = D / 64;                  // elements of d per lane (q loads)
  constexpr int VE = 16 / (int)sizeof(T);      // elements per 16-byte vector
  constexpr int LPR = D / VE;                  // lanes per value row in the weighted sum
  constexpr int RS = 64 / LPR;                 // value rows per step
  typedef T vecT __attribute__((ext_vector_type(VE)));
  extern __shared__ float gc_sc[];             // [SL][N] chunk scores
  __shared__ float qs[SL][D];                  // q (attention)
  __shared__ float qts[SL][D];                 // q~ (scores)
  __shared__ float ps[NW][128];                // one chunk's probabilities per wave (C <= 128)
  __shared__ float sl[SL][64];                 // selected scores, slot order
  __shared__ float wls[SL][64];                // selected weights, slot order
  __shared__ int il[SL][64];                   // selected chunks, slot order (ascending)
  __shared__ int scnt[SL];                     // selected count
  __shared__ int redi[2][W];                   // row-wide counts (W > 1), double-buffered
  __shared__ float red[W > 1 ? W : 1][D];      // the waves' partial outputs (W > 1)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = W == 1 ? wave : 0;          // this wave's row in the workgroup
  const int part = W == 1 ? 0 : wave;          // this wave's share of the row
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const size_t row = (size_t)blockIdx.x * SL + slot;
  // W == 1: a wave past the last row leaves (its row-mates never wait for it).  W > 1: the grid
  // holds exactly one workgroup per row.
  if (W == 1 && row >= (size_t)a.B * a.H * a.L) return;
  float* sc = gc_sc + (size_t)slot * a.N;
  // A wave's own LDS writes, visible to its other lanes.
  auto wsync = [] {
    __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  };
  // The row's LDS writes, visible to every wave of the row.
  auto rsync = [&] {
    if constexpr (W == 1) wsync();
    else __syncthreads();
  };
  int par = 0;
  // Sum of an integer over the row's threads.
  auto row_sum = [&](int c) -> int {
    int s = (int)wave_sum((float)c);           // exact: counts stay below 2^24
    if constexpr (W > 1) {
      if (lane == 0) redi[par][wave] = s;
      __syncthreads();
      s = 0;
#pragma unroll
      for (int u = 0; u < W; ++u) s += redi[par][u];
      par ^= 1;                                // the next call writes the other buffer
    }
    return s;
  };
  const int bh = (int)(row / a.L), i0 = (int)(row % a.L);
  const int b = bh / a.H, h = bh % a.H;
  const size_t kvp = (size_t)b * (a.H / a.G) + h / a.G;
  const int C = a.C;
  const int nc = i0 / C + 1;                   // causal chunks; the last one holds the query
  const float scale = a.scale;

  // q and q~ = round(q + W_up t): the offset and the sum in fp32, one rounding to the dtype.
  if (part == 0) {
    const T* qrow = static_cast<const T*>(a.q) + row * D;
#pragma unroll
    for (int u = 0; u < EPL; ++u) {
      const int e = lane + 64 * u;
      const float qv = to_f32(qrow[e]);
      float qt = qv;
      if (a.r > 0) {
        const float* t = a.tcode + ((size_t)b * a.L + i0) * a.tstride;
        const T* wu = static_cast<const T*>(a.w_up) + (size_t)(h * D + e) * a.r;
        float dq = 0.f;
        if (a.r % VE == 0) {
          for (int c = 0; c < a.r; c += VE) {
            const vecT x = *reinterpret_cast<const vecT*>(wu + c);
#pragma unroll
            for (int z = 0; z < VE; ++z) dq = fmaf(to_f32(x[z]), t[c + z], dq);
          }
        } else {
          for (int c = 0; c < a.r; ++c) dq = fmaf(to_f32(wu[c]), t[c], dq);
        }
        qt = to_f32(from_f32<T>(qv + dq));
      }
      qs[slot][e] = qv;
      qts[slot][e] = qt;
    }
  }
  rsync();

  // Scores sigma_j = q~ . lmk_j of the causal chunks, fp32; threads over chunks.
  const T* lm = static_cast<const T*>(a.lmk) + kvp * a.N * D;
  for (int j = part * 64 + lane; j < nc; j += 64 * W) {
    const vecT* lr = reinterpret_cast<const vecT*>(lm + (size_t)j * D);
    float s = 0.f;
#pragma unroll 4
    for (int v = 0; v < D / VE; ++v) {
      const vecT x = lr[v];
#pragma unroll
      for (int z = 0; z < VE; ++z) s = fmaf(to_f32(x[z]), qts[slot][v * VE + z], s);
    }
    sc[j] = s;
  }
  rsync();

  // Top-k: the own chunk nc - 1 forced in (when asked and there are earlier ones) plus the top
  // k1 of the n1 others; ties to the smaller index.
  const bool fl = a.force_local && nc > 1;
  const int n1 = fl ? nc - 1 : nc, k1 = fl ? a.k - 1 : a.k;
  uint32_t th = 0u;                            // every finite score's key is above 0
  int meq = n1;                                // entries equal to th to take, earliest first
  if (n1 > k1 && k1 > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = th | (1u << bit);
      int c = 0;
      for (int j = part * 64 + lane; j < n1; j += 64 * W) c += f32_key(sc[j]) >= cand ? 1 : 0;
      if (row_sum(c) >= k1) th = cand;
    }
    int gt = 0;
    for (int j = part * 64 + lane; j < n1; j += 64 * W) gt += f32_key(sc[j]) > th ? 1 : 0;
    meq = k1 - row_sum(gt);
  }
  if (part == 0) {
    int cnt = 0;
    if (k1 > 0) {
      int eqrun = 0;
      for (int base = 0; base < n1 && cnt < k1; base += 64) {
        const int j = base + lane;
        const uint32_t kj = j < n1 ? f32_key(sc[j]) : 0u;
        const bool eq = j < n1 && kj == th;
        const uint64_t be = __ballot(eq);
        const bool s = j < n1 && (kj > th || (eq && eqrun + __popcll(be & below) < meq));
        eqrun += __popcll(be);
        const uint64_t bs = __ballot(s);
        if (s) {
          const int p = cnt + __popcll(bs & below);
          il[slot][p] = j;
          sl[slot][p] = sc[j];
        }
        cnt += __popcll(bs);
      }
    }
    if (fl) {
      if (lane == 0) {
        il[slot][cnt] = nc - 1;
        sl[slot][cnt] = sc[nc - 1];
      }
      ++cnt;
    }
    wsync();
    // Softmax over the selected scores; idx / w out (ascending chunks, -1 / 0 padding).
    const float sv = lane < cnt ? sl[slot][lane] : -INFINITY;
    const float mx = wave_max(sv);
    const float ev = lane < cnt ? expf((sv - mx) * scale) : 0.f;
    const float wsum = wave_sum(ev);
    const float wl = lane < cnt ? ev / wsum : 0.f;
    const int jl = lane < cnt ? il[slot][lane] : -1;
    if (lane < a.k) {
      a.idx[row * a.k + lane] = jl;
      a.w[row * a.k + lane] = wl;
    }
    wls[slot][lane] = wl;
    if (lane == 0) scnt[slot] = cnt;
  }
  // Selection only (no output tensor): the chunk-major MFMA kernels attend afterwards.  Uniform
  // over the workgroup, so no wave is left waiting at a barrier.
  if (a.o == nullptr) return;
  rsync();

  // The row's selected chunks, split over its waves: softmax over each chunk's visible keys,
  // the weighted sum of its values.
  const int cnt = scnt[slot];
  const int sub = lane / LPR, dv = lane % LPR;
  float acc[VE];
#pragma unroll
  for (int z = 0; z < VE; ++z) acc[z] = 0.f;
  const T* kbase = static_cast<const T*>(a.key) + kvp * a.L * D;
  const T* vbase = static_cast<const T*>(a.val) + kvp * a.L * D + dv * VE;
  for (int s = part; s < cnt; s += W) {
    const int j = il[slot][s];
    const float wj = wls[slot][s];
    const int lo = j * C, nk = min(lo + C, i0 + 1) - lo;
    float lmax = -INFINITY;
    for (int t = lane; t < nk; t += 64) {
      const vecT* kr = reinterpret_cast<const vecT*>(kbase + (size_t)(lo + t) * D);
      float s2 = 0.f;
#pragma unroll 4
      for (int v = 0; v < D / VE; ++v) {
        const vecT x = kr[v];
#pragma unroll
        for (int z = 0; z < VE; ++z) s2 = fmaf(to_f32(x[z]), qs[slot][v * VE + z], s2);
      }
      s2 *= scale;
      ps[wave][t] = s2;
      lmax = fmaxf(lmax, s2);
    }
    lmax = wave_max(lmax);
    float lsum = 0.f;
    for (int t = lane; t < nk; t += 64) {
      const float p = expf(ps[wave][t] - lmax);
      ps[wave][t] = p;
      lsum += p;
    }
    lsum = wave_sum(lsum);
    wsync();
    const float f = wj / lsum;
#pragma unroll 4
    for (int t = sub; t < nk; t += RS) {
      const float p = ps[wave][t] * f;
      const vecT x = *reinterpret_cast<const vecT*>(vbase + (size_t)(lo + t) * D);
#pragma unroll
      for (int z = 0; z < VE; ++z) acc[z] = fmaf(p, to_f32(x[z]), acc[z]);
    }
    wsync();                                   // ps is rewritten by the next chunk
  }
  // Sum over the value rows a wave took side by side, then over the row's waves.
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int z = 0; z < VE; ++z) acc[z] += shfl_xor_f(acc[z], m);
  if constexpr (W > 1) {
    if (sub == 0)
#pragma unroll
      for (int z = 0; z < VE; ++z) red[wave][dv * VE + z] = acc[z];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int z = 0; z < VE; ++z) {
      float v = 0.f;
#pragma unroll
      for (int u = 0; u < W; ++u) v += red[u][dv * VE + z];
      acc[z] = v;
    }
  }
  if (sub == 0) {
    vecT y;
#pragma unroll
    for (int z = 0; z < VE; ++z) y[z] = from_f32<T>(acc[z]);
    *reinterpret_cast<vecT*>(static_cast<T*>(a.o) + row * D + dv * VE) = y;
  }
}

template <typename T, int D, int W>
hipError_t launch_gchunk_w(const GcArgs& a, size_t rows, hipStream_t st) {
  constexpr int SL = W == 1 ? kGcRows : 1;
  const size_t lds = (size_t)SL * a.N * sizeof(float);
  hipLaunchKernelGGL((gchunk_kernel<T, D, W>), dim3((unsigned)((rows + SL - 1) / SL)),
                     dim3(W == 1 ? 64 * kGcRows : 64 * W), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_gchunk(const GcArgs& a, hipStream_t st) {
  const size_t rows = (size_t)a.B * a.H * a.L;
  if (rows == 0) return hipSuccess;
  if (rows <= (size_t)kGcFewRows) return launch_gchunk_w<T, D, 16>(a, rows, st);
  if (a.N > kGcWideChunks) return launch_gchunk_w<T, D, 4>(a, rows, st);
  return launch_gchunk_w<T, D, 1>(a, rows, st);
}

template hipError_t launch_gchunk<bf16, 64>(const GcArgs&, hipStream_t);
template hipError_t launch_gchunk<bf16, 128>(const GcArgs&, hipStream_t);
template hipError_t launch_gchunk<float, 64>(const GcArgs&, hipStream_t);
template hipError_t launch_gchunk<float, 128>(const GcArgs&, hipStream_t);

}  // namespace hils
