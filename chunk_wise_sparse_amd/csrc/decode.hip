// Decode step: one new token per sequence attends over its key/value cache.
//
// The same method as prefill for a single query at position kv_len-1 (candidates: chunks
// 0..floor((kv_len-1)/C), the last one possibly partial and causally cut at kv_len).  It is
// memory-bound: the step streams every landmark of every (sequence, head) once, then gathers the
// k selected chunks' keys and values once.  Four launches on the caller's stream:
//   scores  - landmark scan, coalesced 16-byte loads, sigma_j = q~ . lmk_j in fp32;
//   select  - exact top-k per (sequence, head) by radix select on order-preserving keys
//             (ties to the smaller chunk index), inter-chunk softmax, ascending output;
//   attend  - one wave per selected chunk: softmax of the raw query over the chunk's visible
//             keys, weighted partial w_j * o_j in fp32;
//   reduce  - o = sum of the partials in slot order (deterministic).
// Method: [HiLS-Attention model page, "Model Description"]; [HiLS Attention explainer
// (molayo1419.me), "Core idea"]; [news page "HiLS Attention Extrapolates 64x ...": per-chunk
// outputs fused by the retrieval scores]; per decode step cost is what the explainer's
// "Numerical results" compares against full attention.
#include <float.h>

#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int kScoreChunksPerBlock = 256;

// Lanes sharing one 16-byte-vector row: reduce over the LPR lanes of a row group.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int mk = LPR / 2; mk >= 1; mk >>= 1) v += shfl_xor_f(v, mk);
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_scores_kernel(const DecodeArgs a) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int LPR = D / VE;          // lanes per landmark row
  constexpr int RPI = 64 / LPR;        // rows per wave iteration
  constexpr int NIT = 64 / RPI;        // iterations for a wave's 64 rows
  const int bh = blockIdx.x, b = bh / a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int n_b = (kvl + kChunk - 1) / kChunk;
  const int base = blockIdx.y * kScoreChunksPerBlock + wave * 64;
  if (base >= n_b) return;
  const int seg = lane % LPR, sub = lane / LPR;
  typedef T vecT __attribute__((ext_vector_type(VE)));
  const vecT qv = *reinterpret_cast<const vecT*>(static_cast<const T*>(a.q_tilde) + (size_t)bh * D + seg * VE);
  float qf[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) qf[e] = to_f32(qv[e]);
  const T* L = static_cast<const T*>(a.lmk) + (size_t)bh * a.Nmax * D;
  vecT rows[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = base + it * RPI + sub;
    rows[it] = r < n_b ? *reinterpret_cast<const vecT*>(L + (size_t)r * D + seg * VE) : vecT{};
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) s = fmaf(to_f32(rows[it][e]), qf[e], s);
    s = row_sum<LPR>(s);
    const int r = base + it * RPI + sub;
    if (seg == 0 && r < n_b) a.scores[(size_t)bh * a.Nmax + r] = s;
  }
}

// Block-wide exclusive scan of one int per thread (256 threads); also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = scratch[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(256) void decode_select_kernel(const DecodeArgs a) {
  __shared__ int hist[256];
  __shared__ int scratch[8];
  __shared__ int bin_found[2];
  __shared__ float evals[64];
  __shared__ uint32_t kmax_w[4];
  const int bh = blockIdx.x, b = bh / a.H, tid = threadIdx.x;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int n = (kvl + kChunk - 1) / kChunk;
  const int kk = min(a.k, n);
  const float* S = a.scores + (size_t)bh * a.Nmax;

  // Radix select of the kk-th largest key, 8 bits at a time from the top.
  uint32_t prefix = 0u, pmask = 0u;
  int krem = kk;
  uint32_t kmax = 0u;
  for (int dg = 3; dg >= 0; --dg) {
    hist[tid] = 0;
    __syncthreads();
    const int sh = dg * 8;
    for (int x = tid; x < n; x += 256) {
      const uint32_t key = f32_key(S[x]);
      if (dg == 3) kmax = max(kmax, key);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & 255u], 1);
    }
    __syncthreads();
    // suffix count for bin tid: sum of hist[tid..255]
    const int hv = hist[255 - tid];
    int tot;
    const int ex = block_exclusive_scan(hv, scratch, tot);   // over reversed bins
    const int suffix_incl = ex + hv;                         // bins >= 255 - tid
    const int suffix_excl = ex;                              // bins >  255 - tid
    if (suffix_incl >= krem && suffix_excl < krem) {
      bin_found[0] = 255 - tid;
      bin_found[1] = suffix_excl;
    }
    __syncthreads();
    const int bsel = bin_found[0];
    krem -= bin_found[1];
    prefix |= (uint32_t)bsel << sh;
    pmask |= 255u << sh;
    __syncthreads();
  }
  const uint32_t theta = prefix;   // key of the kk-th largest score; take krem entries == theta

  // Global maximum (always selected) for the softmax.
  uint32_t km = kmax;
#pragma unroll
  for (int mk = 32; mk >= 1; mk >>= 1) km = max(km, shfl_xor_u(km, mk));
  if ((tid & 63) == 0) kmax_w[tid >> 6] = km;
  __syncthreads();
  const float smax = key_f32(max(max(kmax_w[0], kmax_w[1]), max(kmax_w[2], kmax_w[3])));

  // Each thread owns a contiguous index segment; ties at theta go to the smallest indices.
  const int P = (n + 255) / 256;
  const int lo = tid * P, hi = min(n, lo + P);
  int eq = 0;
  for (int x = lo; x < hi; ++x) eq += f32_key(S[x]) == theta ? 1 : 0;
  int tot;
  int eq_rank = block_exclusive_scan(eq, scratch, tot);
  int nsel = 0;
  {
    int er = eq_rank;
    for (int x = lo; x < hi; ++x) {
      const uint32_t key = f32_key(S[x]);
      bool s = key > theta;
      if (key == theta) { s = er < krem; ++er; }
      nsel += s ? 1 : 0;
    }
  }
  int pos = block_exclusive_scan(nsel, scratch, tot);
  const float zs = a.scale * 1.4426950408889634f;
  int32_t* I = a.idx + (size_t)bh * a.k;
  float* W = a.w + (size_t)bh * a.k;
  {
    int er = eq_rank;
    for (int x = lo; x < hi; ++x) {
      const float sv = S[x];
      const uint32_t key = f32_key(sv);
      bool s = key > theta;
      if (key == theta) { s = er < krem; ++er; }
      if (s) {
        I[pos] = x;
        evals[pos] = exp2f((sv - smax) * zs);
        ++pos;
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    const float e = tid < kk ? evals[tid] : 0.f;
    const float sum = wave_sum(e);
    if (tid < kk) W[tid] = e / sum;
    else if (tid < a.k) { W[tid] = 0.f; I[tid] = -1; }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_attend_kernel(const DecodeArgs a) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int LPR = D / VE;
  constexpr int RPI = 64 / LPR;
  constexpr int NIT = 64 / RPI;
  __shared__ float sp[4][64];
  const int bh = blockIdx.x, b = bh / a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int u = blockIdx.y * 4 + wave;
  // Every wave reaches every barrier; idle slots (u >= k, or padding j < 0) do no loads.
  const bool active = u < a.k;
  const int j = active ? a.idx[(size_t)bh * a.k + u] : -1;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const bool live = j >= 0 && j * kChunk < kvl;
  const int n_vis = live ? min(kChunk, kvl - j * kChunk) : 0;
  const int seg = lane % LPR, sub = lane / LPR;
  typedef T vecT __attribute__((ext_vector_type(VE)));
  const vecT qv = *reinterpret_cast<const vecT*>(static_cast<const T*>(a.q) + (size_t)bh * D + seg * VE);
  float qf[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) qf[e] = to_f32(qv[e]);
  const size_t row0 = (size_t)bh * a.Lmax + (size_t)(live ? j : 0) * kChunk;
  const T* Kc = static_cast<const T*>(a.k_cache) + row0 * D;
  const T* Vc = static_cast<const T*>(a.v_cache) + row0 * D;
  vecT kr[NIT], vr[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = it * RPI + sub;
    kr[it] = r < n_vis ? *reinterpret_cast<const vecT*>(Kc + (size_t)r * D + seg * VE) : vecT{};
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = it * RPI + sub;
    vr[it] = r < n_vis ? *reinterpret_cast<const vecT*>(Vc + (size_t)r * D + seg * VE) : vecT{};
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) s = fmaf(to_f32(kr[it][e]), qf[e], s);
    s = row_sum<LPR>(s);
    const int r = it * RPI + sub;
    if (seg == 0) sp[wave][r] = r < n_vis ? s : -INFINITY;
  }
  __syncthreads();
  const float zs = a.scale * 1.4426950408889634f;
  const float sv = sp[wave][lane];
  const float mx = live ? wave_max(sv) : 0.f;
  const float p = live ? exp2f((sv - mx) * zs) : 0.f;
  const float l = wave_sum(p);
  const float f = live ? a.w[(size_t)bh * a.k + u] / l : 0.f;
  __syncthreads();
  sp[wave][lane] = p * f;
  __syncthreads();
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = it * RPI + sub;
    const float pr = sp[wave][r];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = fmaf(pr, to_f32(vr[it][e]), acc[e]);
  }
#pragma unroll
  for (int mk = LPR; mk < 64; mk <<= 1) {
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] += shfl_xor_f(acc[e], mk);
  }
  if (active && lane < LPR) {
    float* part = a.partial + ((size_t)bh * a.k + u) * D;
#pragma unroll
    for (int e = 0; e < VE; ++e) part[seg * VE + e] = acc[e];
  }
}

template <typename T, int D>
__global__ void decode_reduce_kernel(const DecodeArgs a) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* P = a.partial + (size_t)bh * a.k * D + d;
  float s = 0.f;
  for (int u = 0; u < a.k; ++u) s += P[(size_t)u * D];
  static_cast<T*>(a.o)[(size_t)bh * D + d] = from_f32<T>(s);
}

template <typename T, int D>
hipError_t launch_decode_scores(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.B * a.H, (a.Nmax + kScoreChunksPerBlock - 1) / kScoreChunksPerBlock);
  hipLaunchKernelGGL((decode_scores_kernel<T, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_decode_select(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(decode_select_kernel, dim3(a.B * a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t launch_decode_attend(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.B * a.H, (a.k + 3) / 4);
  hipLaunchKernelGGL((decode_attend_kernel<T, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(a.B * a.H), dim3(D), 0, st, a);
  return hipGetLastError();
}

#define HILS_DECODE_INST(T, D)                                                      \
  template hipError_t launch_decode_scores<T, D>(const DecodeArgs&, hipStream_t); \
  template hipError_t launch_decode_attend<T, D>(const DecodeArgs&, hipStream_t); \
  template hipError_t launch_decode_reduce<T, D>(const DecodeArgs&, hipStream_t);
HILS_DECODE_INST(bf16, 64)
HILS_DECODE_INST(bf16, 128)
HILS_DECODE_INST(float, 64)
HILS_DECODE_INST(float, 128)

}  // namespace hils
