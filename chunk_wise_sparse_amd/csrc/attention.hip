// Intra-chunk attention and fusion for prefill, one workgroup per (batch, head, 64-query tile).
//
// Method: [HiLS Attention explainer (molayo1419.me), "Core idea", level 2] ordinary softmax
// attention over the tokens of each selected chunk; ["HiLS Attention Extrapolates 64x at 90%
// Retrieval Accuracy"] each chunk is attended independently and the per-chunk outputs are summed
// with the inter-chunk weights.  Because every chunk's softmax is normalised on its own, the
// fused output is sum_j (w_j / l_j) * sum_t exp(a_t - m_j) v_t: no rescaling across chunks.
//
// Kernel ("load the union once", the pages' one-load-multiple-compute idea, designed afresh for
// wave64/MFMA): the 64 queries of a tile share the union of their selected chunks.  Each union
// chunk's K (row-major) and V (transposed) are staged once in LDS and used by all four waves.
// Wave w owns queries 16w..16w+15 and skips a chunk that none of its queries selected.
//   S^T[key][q] = K . Q^T : A = K rows from LDS, B = raw q in registers;
//   lane (m, g) then holds query m and keys 16*kb + 4g + rr of the chunk;
//   O^T[d][q] += V^T . P'^T : A = V^T rows from LDS, B = P' = p * (w_j / l_j) from registers.
#include <float.h>

#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T, int D>
struct AttnSmem {
  static constexpr int LDK = D + 16 / (int)sizeof(T);    // K row stride (elements)
  static constexpr int LDV = 64 + 8 / (int)sizeof(T) * 2;  // V^T row stride (elements)
  T k[64 * LDK];
  T vt[D * LDV];
  int32_t idx[64 * 64];
  float w[64 * 64];
  uint32_t bitmap[2048];
};

// Fragment of a V^T row (64 keys) for PV step st: key slots match the S^T output layout,
// i.e. slot z of group g holds key 16*(i/4) + 4g + i%4 with i = st*KPL + z.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag vt_frag(const T* row, int g, int st);
template <>
__device__ __forceinline__ bf16x8 vt_frag<bf16>(const bf16* row, int g, int st) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * st + 4 * g);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * st + 16 + 4 * g);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <>
__device__ __forceinline__ float vt_frag<float>(const float* row, int g, int st) {
  return row[16 * (st >> 2) + 4 * g + (st & 3)];
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void chunk_attention_kernel(const AttnArgs a) {
  typedef AttnSmem<T, D> Smem;
  constexpr int LDK = Smem::LDK, LDV = Smem::LDV;
  constexpr int KPL = Mfma<T>::KPL;
  constexpr int NF = D / 4 / KPL;            // QK^T steps over d
  constexpr int NP = 64 / Mfma<T>::K;        // PV steps over the 64 keys
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int VPR = D / VE;                // 16-byte vectors per row
  constexpr int NV = 64 * VPR / 256;         // vectors per thread, for K and for V
  constexpr int KPT = NV;                    // V: consecutive keys per thread
  __shared__ Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const uint32_t total = (uint32_t)a.B * a.H * a.N;
  const uint32_t tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / a.N;
  const int c = (int)(tile % a.N);
  const int ql = wave * 16 + m;              // query within the tile
  const int qpos = c * 64 + ql;
  const int k = a.topk;
  const T* Kb = static_cast<const T*>(a.key) + (size_t)bh * a.L * D;
  const T* Vb = static_cast<const T*>(a.val) + (size_t)bh * a.L * D;

  // Selection of the tile's 64 rows, and the union bitmap.
  const size_t sel0 = ((size_t)bh * a.L + (size_t)c * 64) * k;
  const int nwords = (c + 1 + 31) >> 5;
  for (int x = tid; x < 64 * k; x += 256) {
    sm.idx[x] = a.idx[sel0 + x];
    sm.w[x] = a.w[sel0 + x];
  }
  for (int x = tid; x < nwords; x += 256) sm.bitmap[x] = 0u;
  __syncthreads();
  for (int x = tid; x < 64 * k; x += 256) {
    const int j = sm.idx[x];
    if (j >= 0 && j <= c) atomicOr(&sm.bitmap[j >> 5], 1u << (j & 31));   // causal chunks only
  }

  // Raw query fragments (contiguous mapping: group g owns d in [g*D/4, (g+1)*D/4)).
  typename Mfma<T>::frag qf[NF];
  {
    const T* qp = static_cast<const T*>(a.q) + ((size_t)bh * a.L + qpos) * D + g * (D / 4);
#pragma unroll
    for (int st = 0; st < NF; ++st) qf[st] = load_frag<T>(qp + st * KPL);
  }
  f32x4 acc_o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc_o[db] = zero4();

  u32x4 kpre[NV], vpre[NV];
  auto load_kv = [&](int j) {
    const T* kc = Kb + (size_t)j * 64 * D;
    const T* vc = Vb + (size_t)j * 64 * D;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = tid + 256 * u;
      kpre[u] = *reinterpret_cast<const u32x4*>(kc + (size_t)(v / VPR) * D + (v % VPR) * VE);
    }
    const int cv = tid % VPR, kg = tid / VPR;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      vpre[u] = *reinterpret_cast<const u32x4*>(vc + (size_t)(kg * KPT + u) * D + cv * VE);
  };
  auto store_kv = [&]() {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = tid + 256 * u;
      *reinterpret_cast<u32x4*>(&sm.k[(v / VPR) * LDK + (v % VPR) * VE]) = kpre[u];
    }
    const int cv = tid % VPR, kg = tid / VPR;
    typedef T rowT __attribute__((ext_vector_type(KPT)));
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      rowT col;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        typedef T vecT __attribute__((ext_vector_type(VE)));
        col[u] = __builtin_bit_cast(vecT, vpre[u])[e];
      }
      *reinterpret_cast<rowT*>(&sm.vt[(cv * VE + e) * LDV + kg * KPT]) = col;
    }
  };

  __syncthreads();
  // Union iterator, identical in every thread: ascending chunk order.
  int wi = 0;
  uint32_t cur = sm.bitmap[0];
  auto next_chunk = [&]() -> int {
    while (cur == 0u && wi + 1 < nwords) cur = sm.bitmap[++wi];
    if (cur == 0u) return -1;
    const int j = wi * 32 + __builtin_ctz(cur);
    cur &= cur - 1u;
    return j;
  };

  const float zs = a.scale * 1.4426950408889634f;
  int ptr = 0;   // next unconsumed entry of this lane's query in its ascending selection
  int j = next_chunk();
  if (j >= 0) load_kv(j);
  while (j >= 0) {
    const int jn = next_chunk();
    __syncthreads();
    store_kv();
    __syncthreads();
    if (jn >= 0) load_kv(jn);

    const bool sel = ptr < k && sm.idx[ql * k + ptr] == j;
    const float wq = sel ? sm.w[ql * k + ptr] : 0.f;
    ptr += sel ? 1 : 0;
    if (__any(sel)) {
      float s[16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f32x4 acc = zero4();
        const T* krow = &sm.k[(kb * 16 + m) * LDK + g * (D / 4)];
#pragma unroll
        for (int st = 0; st < NF; ++st) acc = Mfma<T>::mma(load_frag<T>(krow + st * KPL), qf[st], acc);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int kl = kb * 16 + 4 * g + rr;
          s[kb * 4 + rr] = (j == c && kl > ql) ? -INFINITY : acc[rr];
        }
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = col_max(mx);
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = exp2f((s[i] - mx) * zs);
        l += s[i];
      }
      l = col_sum(l);
      const float f = wq / l;
      typename Mfma<T>::frag pf[NP];
#pragma unroll
      for (int st = 0; st < NP; ++st) {
        if constexpr (KPL == 1) {
          pf[st] = s[st] * f;
        } else {
#pragma unroll
          for (int z = 0; z < KPL; ++z) pf[st][z] = bf16_rne(s[st * KPL + z] * f);
        }
      }
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const T* vrow = &sm.vt[(db * 16 + m) * LDV];
#pragma unroll
        for (int st = 0; st < NP; ++st) acc_o[db] = Mfma<T>::mma(vt_frag<T>(vrow, g, st), pf[st], acc_o[db]);
      }
    }
    j = jn;
  }

  // O^T fragments: lane holds query ql and d = 16*db + 4g + rr.
  T* op = static_cast<T*>(a.o) + ((size_t)bh * a.L + qpos) * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    typedef T vec4 __attribute__((ext_vector_type(4)));
    vec4 out;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) out[rr] = from_f32<T>(acc_o[db][rr]);
    *reinterpret_cast<vec4*>(op + db * 16 + 4 * g) = out;
  }
}

template <typename T, int D>
hipError_t launch_chunk_attention(const AttnArgs& a, hipStream_t st) {
  const uint32_t total = (uint32_t)a.B * a.H * a.N;
  hipLaunchKernelGGL((chunk_attention_kernel<T, D>), dim3(total), dim3(256), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_chunk_attention<bf16, 64>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<bf16, 128>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<float, 64>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<float, 128>(const AttnArgs&, hipStream_t);

}  // namespace hils
