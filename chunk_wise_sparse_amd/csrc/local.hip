// Forced local chunk (an option of prefill and decode): the query's own chunk is always
// selected and the other k - 1 slots hold the best-scoring earlier chunks.  The pages do not force
// the own chunk [HiLS-Attention model page, "Model Description": the top-k chunks by score]; a
// serving stack may, so it is offered as a flag.
//
// It runs after the ordinary exact top-k (whatever kernel produced it), per row: if the own chunk
// c is already selected - always the case when every candidate fits in k - the row is left as it
// is ({c} plus the best k - 1 others is then the top-k itself).  Otherwise the top-k holds the k
// best earlier chunks, and {c} plus the best k - 1 of them is that set minus its worst entry
// (lowest score, the larger index among equal scores), plus c.  The kernel recomputes q~ and the
// k + 1 scores it needs, drops the worst entry, appends c (larger than every earlier index, so the
// list stays ascending) and redoes the inter-chunk softmax.  One wave per row.
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T, int D, bool DECODE>
__global__ __launch_bounds__(256) void force_local_kernel(const LocalArgs a) {
  __shared__ float qs[4][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wave;
  const size_t rows = DECODE ? (size_t)a.B * a.H : (size_t)a.B * a.H * a.L;
  if (row >= rows) return;                     // whole wave: no barrier below
  int bh, i;
  const float* t;
  if constexpr (DECODE) {
    bh = (int)row;
    i = min(max(a.kv_len[bh / a.H], 1), a.L) - 1;
    t = a.tcode + (size_t)(bh / a.H) * a.tstride;
  } else {
    bh = (int)(row / a.L);
    i = (int)(row % a.L);
    t = a.tcode + ((size_t)(bh / a.H) * a.L + i) * a.tstride;
  }
  const int c = i >> a.lc, k = a.k, h = bh % a.H;
  if (c + 1 <= k) return;                      // every candidate selected
  int32_t* ip = a.idx + row * k;
  float* wp = a.w + row * k;
  const int j = lane < k ? ip[lane] : -1;
  if (__any(j == c)) return;                   // the own chunk is already in
  // q~ = round_dtype(q + W_up[h] t), as the forward forms it
  const T* q = static_cast<const T*>(a.q) + row * D;
  const T* wu = static_cast<const T*>(a.w_up) + (size_t)h * D * a.r;
  for (int e = lane; e < D; e += 64) {
    float v = to_f32(q[e]);
    if (a.r > 0) {
      float dq = 0.f;
      for (int z = 0; z < a.r; ++z) dq = fmaf(to_f32(wu[(size_t)e * a.r + z]), t[z], dq);
      v = to_f32(from_f32<T>(v + dq));
    }
    qs[wave][e] = v;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const T* lmk = static_cast<const T*>(a.lmk) + (size_t)kv_pair(bh, a.H, a.G) * a.N * D;
  float sig = -INFINITY;
  if (lane < k) {
    const T* lr = lmk + (size_t)j * D;
    float acc = 0.f;
    for (int e = 0; e < D; ++e) acc = fmaf(qs[wave][e], to_f32(lr[e]), acc);
    sig = acc;
  }
  float part = 0.f;
  for (int e = lane; e < D; e += 64) part = fmaf(qs[wave][e], to_f32(lmk[(size_t)c * D + e]), part);
  const float sc = wave_sum(part);
  // the worst selected entry: lowest score, the larger chunk index among equal scores
  const uint64_t comp = lane < k ? ((uint64_t)f32_key(sig) << 32) | (uint32_t)(0xFFFFu - (uint32_t)j) : ~0ull;
  uint64_t mn = comp;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(mn, m);
    mn = o < mn ? o : mn;
  }
  const int pw = __ffsll((unsigned long long)__ballot(comp == mn)) - 1;
  const int src = lane < pw ? lane : min(lane + 1, 63);
  int nj = __shfl(j, src, 64);
  float nsig = __shfl(sig, src, 64);
  if (lane == k - 1) {
    nj = c;
    nsig = sc;
  }
  const float zs = a.scale * 1.4426950408889634f;
  const float mx = wave_max(lane < k ? nsig : -INFINITY);
  const float ev = lane < k ? exp2f((nsig - mx) * zs) : 0.f;
  const float inv = 1.f / wave_sum(ev);
  if (lane < k) {
    ip[lane] = nj;
    wp[lane] = ev * inv;
  }
}

template <typename T, int D>
hipError_t launch_force_local(const LocalArgs& a, bool decode, hipStream_t st) {
  const size_t rows = decode ? (size_t)a.B * a.H : (size_t)a.B * a.H * a.L;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (decode) hipLaunchKernelGGL((force_local_kernel<T, D, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((force_local_kernel<T, D, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_force_local<bf16, 64>(const LocalArgs&, bool, hipStream_t);
template hipError_t launch_force_local<bf16, 128>(const LocalArgs&, bool, hipStream_t);
template hipError_t launch_force_local<float, 64>(const LocalArgs&, bool, hipStream_t);
template hipError_t launch_force_local<float, 128>(const LocalArgs&, bool, hipStream_t);

}  // namespace hils
