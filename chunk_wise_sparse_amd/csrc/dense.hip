// Dense causal attention: the full-attention baseline that HiLS is compared against.
//
// [HiLS Attention explainer (molayo1419.me), "Numerical results"]: prefill and each decode step
// are compared with full attention on the same hardware at 512K tokens.  Full attention is the
// textbook o_i = sum_t softmax_t(scale * q_i . k_t) v_t over every key t <= i (prefill), or over
// the whole cache of kv_len keys (decode).  These kernels compute it on this GPU with the same
// tile machinery as the HiLS prefill, so that the two are compared kernel against kernel.
//
// Prefill (dense_prefill_kernel): a workgroup takes 16*NW consecutive queries of one (batch,
// head), one 16-row MFMA block per wave, and walks every causal 64-key chunk in ascending order;
// each chunk's K and V are staged once in LDS and shared by the waves.  A softmax running over
// the chunks (running maximum m and sum l per row, the accumulator rescaled by exp(m_old - m_new)
// when the maximum grows) gives the exact result after the last chunk.  Groups run longest first.
//
// Decode (dense_decode_split_kernel + dense_decode_reduce_kernel): each (sequence, head) pair's
// cache is split over several workgroups.  A wave streams 64-key tiles with 16-byte coalesced
// loads: lane (ro, dg) of a row segment holds dims dg*VE.. of rows ro + RPL*i; the partial dot
// products are summed over the segment by a butterfly that leaves lane dg with the score of row
// ro + RPL*dg, and the weights go back to the value rows by lane shuffles.  Each workgroup writes
// (m, l, acc[d]) for its span; a second kernel combines the spans in a fixed order.
#include <float.h>

#include "attn_tiles.h"
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void dense_prefill_kernel(const DenseArgs a) {
  constexpr int QG = 16 * NW;
  typedef AttnLayout<T, D> Lay;
  typedef Mfma<T> M;
  constexpr int KPL = M::KPL;
  constexpr int NF = D / 4 / KPL;            // QK^T steps over d
  constexpr int NP = 64 / M::K;              // PV steps over the 64 keys
  constexpr int VE = 16 / (int)sizeof(T);    // elements per 16-byte vector
  constexpr int NT = NW * 64;
  constexpr int NV = 64 * Lay::VPR / NT;     // 16-byte vectors per thread per tensor per chunk
  static_assert(NV >= 1 && (64 * Lay::VPR) % NT == 0, "chunk tile does not split over the threads");
  __shared__ alignas(16) char ks[Lay::KBYTES];
  __shared__ alignas(16) char vs[Lay::VBYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int groups = a.L / QG;
  const uint32_t total = (uint32_t)a.B * a.H * groups;
  const uint32_t gid = xcd_remap(blockIdx.x, total);
  const int bh = gid / groups;
  const int q0 = (groups - 1 - (int)(gid % groups)) * QG;   // longest groups first
  const int c_last = (q0 + QG - 1) >> 6;
  const T* Kb = static_cast<const T*>(a.key) + (size_t)kv_pair(bh, a.H, a.G) * a.L * D;
  const T* Vb = static_cast<const T*>(a.val) + (size_t)kv_pair(bh, a.H, a.G) * a.L * D;
  const size_t row0 = (size_t)bh * a.L;

  const int qpos = q0 + 16 * wave + m, crow = qpos >> 6;
  typename M::frag qf[NF];
  {
    const T* qp = static_cast<const T*>(a.q) + (row0 + qpos) * D + g * (D / 4);
#pragma unroll
    for (int st = 0; st < NF; ++st) qf[st] = load_frag<T>(qp + st * KPL);
  }
#pragma unroll
  for (int st = 0; st < NF; ++st) asm volatile("" ::"v"(qf[st]));
  f32x4 acc_o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc_o[db] = zero4();
  float mrun = -INFINITY, lrun = 0.f;        // per row, in log2 units

  // K element e of row `row`: bf16 rows use the XOR-permuted layout, fp32 rows are padded.
  auto koff = [&](int row, int e) -> int {
    if constexpr (sizeof(T) == 2) return BlockKLayout<D>::off(row, e / VE);
    else return row * Lay::KLD + e * 4;
  };
  auto load_kv = [&](int j, u32x4 (&kr)[NV], u32x4 (&vr)[NV]) {
    const T* kc = Kb + (size_t)j * 64 * D;
    const T* vc = Vb + (size_t)j * 64 * D;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = tid + NT * u;
      kr[u] = *reinterpret_cast<const u32x4*>(kc + (size_t)v * VE);
      vr[u] = *reinterpret_cast<const u32x4*>(vc + (size_t)v * VE);
    }
  };
  auto store_kv = [&](const u32x4 (&kr)[NV], const u32x4 (&vr)[NV]) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = tid + NT * u;
      const int row = v / Lay::VPR, p = v % Lay::VPR;
      *reinterpret_cast<u32x4*>(ks + koff(row, p * VE)) = kr[u];
      const int e = p * VE;
      *reinterpret_cast<u32x4*>(vs + (e >> 4) * Lay::VDB + row * (16 * (int)sizeof(T)) +
                                (e & 15) * (int)sizeof(T)) = vr[u];
    }
  };

  const float zs = a.scale * 1.4426950408889634f;
  auto compute = [&](int j) {
    if (j > crow) return;                    // wave-uniform: the block's rows share a chunk
    float sv[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = zero4();
#pragma unroll
      for (int st = 0; st < NF; ++st)
        acc = M::mma(load_frag<T>(reinterpret_cast<const T*>(ks + koff(kb * 16 + m, g * (D / 4) + st * KPL))),
                     qf[st], acc);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sv[kb * 4 + rr] = acc[rr];
    }
    if (j == crow) {
      const int ql = qpos & 63;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (kb * 16 + 4 * g + rr > ql) sv[kb * 4 + rr] = -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
    const float mnew = fmaxf(mrun, col_max(mx) * zs);   // finite: the row sees key qpos
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], zs, -mnew));
      l += sv[i];
    }
    lrun = fmaf(lrun, alpha, col_sum(l));
    mrun = mnew;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc_o[db] *= alpha;
    typename M::frag pf[NP];
#pragma unroll
    for (int st = 0; st < NP; ++st) {
      if constexpr (KPL == 1) {
        pf[st] = sv[st];
      } else {
#pragma unroll
        for (int z = 0; z < KPL; ++z) pf[st][z] = bf16_rne(sv[st * KPL + z]);
      }
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int st = 0; st < NP; ++st) {
        typename M::frag va;
        if constexpr (KPL == 1) va = v_frag_f32<Lay::VDB>(vs, m, g, db, st);
        else va = v_frag_bf16<Lay::VDB>(vs, m, g, db, st);
        acc_o[db] = M::mma(va, pf[st], acc_o[db]);
      }
  };

  // compute c_t; barrier; the registers holding c_{t+1} go to LDS and c_{t+2} is loaded into
  // them; barrier.  Loads past the last chunk repeat it, so wait counts stay exact.
  u32x4 kr[NV], vr[NV];
  load_kv(0, kr, vr);
  store_kv(kr, vr);
  load_kv(min(1, c_last), kr, vr);
  __syncthreads();
  for (int j = 0; j <= c_last; ++j) {
    compute(j);
    __syncthreads();
    store_kv(kr, vr);
    load_kv(min(j + 2, c_last), kr, vr);
    __syncthreads();
  }

  const float inv = 1.0f / lrun;
  T* op = static_cast<T*>(a.o) + (row0 + qpos) * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    typedef T vec4 __attribute__((ext_vector_type(4)));
    vec4 out;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) out[rr] = from_f32<T>(acc_o[db][rr] * inv);
    *reinterpret_cast<vec4*>(op + db * 16 + 4 * g) = out;
  }
}

// ------------------------------------------------------------------------------------------
// Decode.
// ------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void dense_decode_split_kernel(const DenseDecodeArgs a) {
  constexpr int VE = 16 / (int)sizeof(T);   // elements per 16-byte vector
  constexpr int LPR = D / VE;               // lanes per row
  constexpr int RPL = 64 / LPR;             // rows per load instruction
  constexpr int NI = LPR;                   // load instructions per 64-key tile (= 64 / RPL)
  typedef T vecT __attribute__((ext_vector_type(VE)));
  __shared__ float wm[4], wl[4];
  __shared__ float wacc[4][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ro = lane / LPR, dg = lane % LPR;
  const int pair = blockIdx.x, split = blockIdx.y, S = gridDim.y;
  const int kvl = min(max(a.kv_len[pair / a.H], 1), a.Lmax);
  const int ntiles = (kvl + 63) / 64;
  const int tps = (ntiles + S - 1) / S;
  const int t0 = split * tps, t1 = min(t0 + tps, ntiles);
  const size_t kvbase = (size_t)kv_pair(pair, a.H, a.G) * a.Lmax * D;
  const T* Kc = static_cast<const T*>(a.k_cache) + kvbase + dg * VE;
  const T* Vc = static_cast<const T*>(a.v_cache) + kvbase + dg * VE;

  const float zs = a.scale * 1.4426950408889634f;
  float qv[VE];
  {
    const vecT x = *reinterpret_cast<const vecT*>(static_cast<const T*>(a.q) + (size_t)pair * D + dg * VE);
#pragma unroll
    for (int e = 0; e < VE; ++e) qv[e] = to_f32(x[e]) * zs;
  }
  float mrun = -INFINITY, lrun = 0.f, acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;

  for (int tile = t0 + wave; tile < t1; tile += 4) {
    const int base = tile * 64;
    vecT kx[NI], vx[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = base + ro + RPL * i;
      if (row < kvl) {
        kx[i] = *reinterpret_cast<const vecT*>(Kc + (size_t)row * D);
        vx[i] = *reinterpret_cast<const vecT*>(Vc + (size_t)row * D);
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) kx[i][e] = vx[i][e] = static_cast<T>(0.f);
      }
    }
    float part[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) s = fmaf(qv[e], to_f32(kx[i][e]), s);
      part[i] = s;
    }
    // Butterfly over the LPR lanes of the segment: positions 0..b-1 keep the row indices whose
    // bit b matches dg's; after the last step part[0] is the score of row ro + RPL * dg.
#pragma unroll
    for (int b = NI / 2; b >= 1; b >>= 1) {
      const bool hi = (dg & b) != 0;
#pragma unroll
      for (int p = 0; p < b; ++p) {
        const float send = hi ? part[p] : part[p + b];
        const float keep = hi ? part[p + b] : part[p];
        part[p] = keep + shfl_xor_f(send, b);
      }
    }
    const int myrow = base + ro + RPL * dg;
    const float s = myrow < kvl ? part[0] : -INFINITY;
    const float mnew = fmaxf(mrun, wave_max(s));            // finite: row base is < kvl
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    const float p = __builtin_amdgcn_exp2f(s - mnew);
    lrun = fmaf(lrun, alpha, wave_sum(p));
    mrun = mnew;
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float pr = __shfl(p, ro * LPR + i, 64);          // weight of row ro + RPL * i
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = fmaf(pr, to_f32(vx[i][e]), acc[e]);
    }
  }
  // Sum the RPL row offsets (lanes with equal dg), then the four waves through LDS.
#pragma unroll
  for (int b = LPR; b < 64; b <<= 1)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] += shfl_xor_f(acc[e], b);
  if (lane == 0) {
    wm[wave] = mrun;
    wl[wave] = lrun;
  }
  if (ro == 0) {
#pragma unroll
    for (int e = 0; e < VE; ++e) wacc[wave][dg * VE + e] = acc[e];
  }
  __syncthreads();
  float* out = a.partial + ((size_t)pair * S + split) * (D + 2);
  const float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  for (int x = tid; x < D; x += 256) {
    float v = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) v = fmaf(wacc[w][x], __builtin_amdgcn_exp2f(wm[w] - M), v);
    }
    out[2 + x] = v;
  }
  if (tid == 0) {
    float l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) l = fmaf(wl[w], __builtin_amdgcn_exp2f(wm[w] - M), l);
    }
    out[0] = M;
    out[1] = l;
  }
}

// o = sum over spans s of acc_s * exp2(m_s - M) / sum_s l_s * exp2(m_s - M), spans in order.
template <typename T, int D>
__global__ __launch_bounds__(D) void dense_decode_reduce_kernel(const DenseDecodeArgs a, int S) {
  const int pair = blockIdx.x, x = threadIdx.x;
  const float* P = a.partial + (size_t)pair * S * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, P[(size_t)s * (D + 2)]);
  float l = 0.f, v = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ms = P[(size_t)s * (D + 2)];
    if (ms == -INFINITY) continue;           // a span past the pair's cache
    const float f = __builtin_amdgcn_exp2f(ms - M);
    l = fmaf(P[(size_t)s * (D + 2) + 1], f, l);
    v = fmaf(P[(size_t)s * (D + 2) + 2 + x], f, v);
  }
  static_cast<T*>(a.o)[(size_t)pair * D + x] = from_f32<T>(v / l);
}

// ------------------------------------------------------------------------------------------
// Launchers.
// ------------------------------------------------------------------------------------------
template <typename T, int D>
hipError_t launch_dense_prefill(const DenseArgs& a, hipStream_t st) {
  const uint32_t bhs = (uint32_t)a.B * a.H;
  if (a.L % 128 == 0)
    hipLaunchKernelGGL((dense_prefill_kernel<T, D, 8>), dim3(bhs * (a.L / 128)), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((dense_prefill_kernel<T, D, 4>), dim3(bhs * (a.L / 64)), dim3(256), 0, st, a);
  return hipGetLastError();
}

int dense_decode_splits(int pairs, int lmax) {
  const int ntiles = (lmax + 63) / 64;
  int s = (4096 + pairs - 1) / pairs;        // about 4096 workgroups in all
  s = min(s, max(1, ntiles / 8));            // at least 8 tiles (two per wave) per span
  return max(1, min(s, 1024));
}

template <typename T, int D>
hipError_t launch_dense_decode(const DenseDecodeArgs& a, hipStream_t st) {
  const int pairs = a.B * a.H;
  const int S = dense_decode_splits(pairs, a.Lmax);
  hipLaunchKernelGGL((dense_decode_split_kernel<T, D>), dim3(pairs, S), dim3(256), 0, st, a);
  hipLaunchKernelGGL((dense_decode_reduce_kernel<T, D>), dim3(pairs), dim3(D), 0, st, a, S);
  return hipGetLastError();
}

template hipError_t launch_dense_prefill<bf16, 64>(const DenseArgs&, hipStream_t);
template hipError_t launch_dense_prefill<bf16, 128>(const DenseArgs&, hipStream_t);
template hipError_t launch_dense_prefill<float, 64>(const DenseArgs&, hipStream_t);
template hipError_t launch_dense_prefill<float, 128>(const DenseArgs&, hipStream_t);
template hipError_t launch_dense_decode<bf16, 64>(const DenseDecodeArgs&, hipStream_t);
template hipError_t launch_dense_decode<bf16, 128>(const DenseDecodeArgs&, hipStream_t);
template hipError_t launch_dense_decode<float, 64>(const DenseDecodeArgs&, hipStream_t);
template hipError_t launch_dense_decode<float, 128>(const DenseDecodeArgs&, hipStream_t);

}  // namespace hils
