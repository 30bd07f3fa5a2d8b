// HiLS for chunk sizes C other than 64 (32 and 128): prefill rows and decode steps, one wave per
// query row.  The steps are the method's [HiLS-Attention model page, "Model Description"; HiLS
// Attention explainer (molayo1419.me), "Core idea" and "Engineering details"]: q~ = q + W_up t
// (Q-Cal), a score per causal chunk against its landmark key, the top-k chunks (ties to the
// smaller index; with the forced local chunk, the own chunk and the top k - 1 earlier ones), a
// softmax over their scores, and each chunk's causal softmax attention fused by those weights.
//
// The 64-key kernels tie their tiles to one 64-key chunk (a 64-query tile shares one candidate
// set, a chunk is one MFMA tile); this path has no such tie and no MFMA: the wave keeps the
// row's scores in LDS (up to 8192 chunks), finds the k-th largest by bisection over the
// order-preserving 32-bit keys with wave-wide counts, takes the keys above it and the earliest
// equal ones in chunk order, and then walks the selected chunks, C keys at a time.  fp32
// arithmetic throughout; q~ and the output are rounded once to the dtype.
#include "gchunk.h"
#include "hils_device.h"

namespace hils {

constexpr int kGcWaves = 2;                    // waves (rows) per workgroup

template <typename T, int D>
__global__ __launch_bounds__(64 * kGcWaves) void gchunk_kernel(const GcArgs a) {
  constexpr int EPL = D / 64;                  // elements of d per lane
  constexpr int VE = 16 / (int)sizeof(T);      // elements per 16-byte vector
  typedef T vecT __attribute__((ext_vector_type(VE)));
  __shared__ float sc[kGcWaves][kGcMaxChunks]; // the row's chunk scores
  __shared__ float qs[kGcWaves][D];            // q (attention)
  __shared__ float qts[kGcWaves][D];           // q~ (scores)
  __shared__ float ps[kGcWaves][128];          // one chunk's probabilities (C <= 128)
  __shared__ float sl[kGcWaves][64];           // selected scores, slot order
  __shared__ int il[kGcWaves][64];             // selected chunks, slot order (ascending)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const size_t row = (size_t)blockIdx.x * kGcWaves + wave;
  if (row >= (size_t)a.B * a.H * a.Lq) return;  // wave-uniform; the waves never synchronise
  // A wave's own LDS writes, visible to its other lanes.
  auto wsync = [] {
    __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
  };
  const int bh = (int)(row / a.Lq), i0 = (int)(row % a.Lq);
  const int b = bh / a.H, h = bh % a.H;
  const size_t kvp = (size_t)b * (a.H / a.G) + h / a.G;
  const int pos = a.kv_len ? min(max(a.kv_len[b], 1), a.Lkv) - 1 : i0;
  const int C = a.C;
  const int nc = pos / C + 1;                  // causal chunks; the last one holds the query
  const float scale = a.scale;

  // q and q~ = round(q + W_up t): the offset and the sum in fp32, one rounding to the dtype.
  const T* qrow = static_cast<const T*>(a.q) + row * D;
#pragma unroll
  for (int u = 0; u < EPL; ++u) {
    const int e = lane + 64 * u;
    const float qv = to_f32(qrow[e]);
    float qt = qv;
    if (a.r > 0) {
      const float* t = a.tcode + (size_t)(a.kv_len ? b : b * a.Lq + i0) * a.tstride;
      const T* wu = static_cast<const T*>(a.w_up) + (size_t)(h * D + e) * a.r;
      float dq = 0.f;
      for (int c = 0; c < a.r; ++c) dq = fmaf(to_f32(wu[c]), t[c], dq);
      qt = to_f32(from_f32<T>(qv + dq));
    }
    qs[wave][e] = qv;
    qts[wave][e] = qt;
  }
  wsync();

  // Scores sigma_j = q~ . lmk_j of the causal chunks, fp32.
  const T* lm = static_cast<const T*>(a.lmk) + kvp * a.N * D;
  for (int j = lane; j < nc; j += 64) {
    const vecT* lr = reinterpret_cast<const vecT*>(lm + (size_t)j * D);
    float s = 0.f;
#pragma unroll 4
    for (int v = 0; v < D / VE; ++v) {
      const vecT x = lr[v];
#pragma unroll
      for (int z = 0; z < VE; ++z) s = fmaf(to_f32(x[z]), qts[wave][v * VE + z], s);
    }
    sc[wave][j] = s;
  }
  wsync();

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
      for (int j = lane; j < n1; j += 64) c += f32_key(sc[wave][j]) >= cand ? 1 : 0;
      if ((int)wave_sum((float)c) >= k1) th = cand;
    }
    int gt = 0;
    for (int j = lane; j < n1; j += 64) gt += f32_key(sc[wave][j]) > th ? 1 : 0;
    meq = k1 - (int)wave_sum((float)gt);
  }
  int cnt = 0;
  if (k1 > 0) {
    int eqrun = 0;
    for (int base = 0; base < n1; base += 64) {
      const int j = base + lane;
      const uint32_t kj = j < n1 ? f32_key(sc[wave][j]) : 0u;
      const bool eq = j < n1 && kj == th;
      const uint64_t be = __ballot(eq);
      const bool s = j < n1 && (kj > th || (eq && eqrun + __popcll(be & below) < meq));
      eqrun += __popcll(be);
      const uint64_t bs = __ballot(s);
      if (s) {
        const int p = cnt + __popcll(bs & below);
        il[wave][p] = j;
        sl[wave][p] = sc[wave][j];
      }
      cnt += __popcll(bs);
    }
  }
  if (fl) {
    if (lane == 0) {
      il[wave][cnt] = nc - 1;
      sl[wave][cnt] = sc[wave][nc - 1];
    }
    ++cnt;
  }
  wsync();

  // Softmax over the selected scores; idx / w out (ascending chunks, -1 / 0 padding).
  const float sv = lane < cnt ? sl[wave][lane] : -INFINITY;
  const float mx = wave_max(sv);
  const float ev = lane < cnt ? expf((sv - mx) * scale) : 0.f;
  const float wsum = wave_sum(ev);
  const float wl = lane < cnt ? ev / wsum : 0.f;
  const int jl = lane < cnt ? il[wave][lane] : -1;
  if (lane < a.k) {
    a.idx[row * a.k + lane] = jl;
    a.w[row * a.k + lane] = wl;
  }

  // Each selected chunk: softmax over its visible keys, the weighted sum of its values.
  float acc[EPL];
#pragma unroll
  for (int u = 0; u < EPL; ++u) acc[u] = 0.f;
  const T* kbase = static_cast<const T*>(a.key) + kvp * a.Lkv * D;
  const T* vbase = static_cast<const T*>(a.val) + kvp * a.Lkv * D;
  for (int s = 0; s < cnt; ++s) {
    const int j = __shfl(jl, s);
    const float wj = __shfl(wl, s);
    const int lo = j * C, nk = min(lo + C, pos + 1) - lo;
    float lmax = -INFINITY;
    for (int t = lane; t < nk; t += 64) {
      const vecT* kr = reinterpret_cast<const vecT*>(kbase + (size_t)(lo + t) * D);
      float s2 = 0.f;
#pragma unroll 4
      for (int v = 0; v < D / VE; ++v) {
        const vecT x = kr[v];
#pragma unroll
        for (int z = 0; z < VE; ++z) s2 = fmaf(to_f32(x[z]), qs[wave][v * VE + z], s2);
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
    for (int t = 0; t < nk; ++t) {
      const float p = ps[wave][t] * f;
      const T* vr = vbase + (size_t)(lo + t) * D;
#pragma unroll
      for (int u = 0; u < EPL; ++u) acc[u] = fmaf(p, to_f32(vr[lane + 64 * u]), acc[u]);
    }
    wsync();                                   // ps is rewritten by the next chunk
  }
  T* orow = static_cast<T*>(a.o) + row * D;
#pragma unroll
  for (int u = 0; u < EPL; ++u) orow[lane + 64 * u] = from_f32<T>(acc[u]);
}

template <typename T, int D>
hipError_t launch_gchunk(const GcArgs& a, hipStream_t st) {
  const size_t rows = (size_t)a.B * a.H * a.Lq;
  hipLaunchKernelGGL((gchunk_kernel<T, D>), dim3((unsigned)((rows + kGcWaves - 1) / kGcWaves)),
                     dim3(64 * kGcWaves), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_gchunk<bf16, 64>(const GcArgs&, hipStream_t);
template hipError_t launch_gchunk<bf16, 128>(const GcArgs&, hipStream_t);
template hipError_t launch_gchunk<float, 64>(const GcArgs&, hipStream_t);
template hipError_t launch_gchunk<float, 128>(const GcArgs&, hipStream_t);

}  // namespace hils
