// Chunk selection for prefill: Q-Cal, inter-chunk scores against the landmarks, exact top-k and
// the inter-chunk softmax, one workgroup per (batch, head, 64-query tile).
//
// Method: [HiLS-Attention model page, "Model Description"] landmark scores stand in for each
// chunk's attention mass; the top-k chunks are kept; the inter-chunk softmax weights them.
// [HiLS Attention explainer (molayo1419.me), "Engineering details", Q-Cal item] the query used
// for scoring is q + W_up W_down h.
//
// Layout: with C = 64 and a 64-query tile, the tile is exactly one chunk c, so every query of the
// tile has the same candidate set {0..c} and scoring is a GEMM [64 queries x d] x [d x (c+1)].
// Wave w owns queries 16w..16w+15 as the MFMA B operand (kept in registers); landmark tiles of
// 64 chunks are staged in LDS and are the A operand.  Output D[chunk][query]: lane (m, g) holds
// query m of its wave and chunks 16*blk + 4g + rr of the tile (blk, rr = 0..3).
//
// Exact top-k in two passes over the landmarks:
//   pass 1 keeps, per lane, the running maximum of each of its 16*R score slots (slot = position
//          in the tile, and tile parity when R = 2).  The ceil(k/4)-th largest of a lane's slot
//          maxima is a score that at least ceil(k/4) distinct chunks reach, so the minimum of it
//          over the query's four lanes is reached by >= k chunks: a lower bound tau of the
//          k-th largest score.
//   pass 2 recomputes the scores and appends every (score >= tau) to a per-query LDS buffer in
//          ascending chunk order.  If the buffer would overflow, it is cut to its exact top-k and
//          tau is raised to the k-th score (strict from then on, since later chunks lose ties).
//   Final: an exact threshold by bisection on order-preserving score keys picks the top k (ties
//          to the smaller chunk), then the inter-chunk softmax over them; output ascending.
// Pass 1 is skipped when the tile has at most kBufCap candidates (all of them fit the buffer).
#include <float.h>

#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int kBufCap = 128;

// Per-query candidate buffers use odd row strides so the 16 queries of a wave hit distinct banks.
constexpr int kBsStride = kBufCap + 1;   // floats
constexpr int kBjStride = kBufCap + 2;   // uint16

template <typename T, int D>
struct SelectSmem {
  static constexpr int LD = D + 16 / (int)sizeof(T);  // padded row stride (elements)
  T lmk[64 * LD];
  float bs[64 * kBsStride];
  uint16_t bj[64 * kBjStride];
};

// A fragment of a landmark row for MFMA step st.  Lane group g's k-slot z of step st holds
// d = 16*(i/4) + 4g + i%4 with i = st*KPL + z (the layout in which Q-Cal's MFMA delivers q~).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag lmk_frag(const T* row, int g, int st);
template <>
__device__ __forceinline__ bf16x8 lmk_frag<bf16>(const bf16* row, int g, int st) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * st + 4 * g);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * st + 16 + 4 * g);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <>
__device__ __forceinline__ float lmk_frag<float>(const float* row, int g, int st) {
  return row[16 * (st >> 2) + 4 * g + (st & 3)];
}

template <int N>
__device__ __forceinline__ void bitonic_sort_desc(float (&x)[N]) {
#pragma unroll
  for (int kk = 2; kk <= N; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ jj;
        if (l > i) {
          const float a = x[i], b = x[l];
          const bool desc = (i & kk) == 0;
          x[i] = desc ? fmaxf(a, b) : fminf(a, b);
          x[l] = desc ? fminf(a, b) : fmaxf(a, b);
        }
      }
    }
  }
}

__device__ __forceinline__ float col_min(float v) {
  v = fminf(v, shfl_xor_f(v, 16));
  return fminf(v, shfl_xor_f(v, 32));
}

// Exact top-kk of one query's buffer [0, cnt) (ascending chunk index), shared by the query's
// four lanes (groups g = 0..3, each owning a contiguous quarter).  On return, sel[i] marks the
// lane's selected entries, key/jx hold them, and pos[i] is each selected entry's rank in chunk
// order.  Returns the key of the kk-th largest score.
struct TopkResult {
  uint32_t theta;
  int nsel_before;   // selected entries in lower groups
};

constexpr int kSeg = kBufCap / 4;

__device__ __forceinline__ TopkResult buffer_topk(const float* bs, const uint16_t* bj, int cnt,
                                                  int kk, int g, uint32_t (&key)[kSeg],
                                                  int (&jx)[kSeg], uint32_t& selmask) {
  const int P = (cnt + 3) >> 2;
  const int lo = g * P;
  const int nmy = max(0, min(cnt, lo + P) - lo);
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    if (i < nmy) {
      key[i] = f32_key(bs[lo + i]);
      jx[i] = bj[lo + i];
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    } else {
      key[i] = 0u;   // below every finite score's key
      jx[i] = 0;
    }
  }
  kmin = col_min_u(kmin);
  kmax = col_max_u(kmax);
  // theta = largest key with count(key >= theta) >= kk; all keys share the bits above the
  // highest bit where kmin and kmax differ.
  const uint32_t diff = kmin ^ kmax;
  uint32_t theta = kmax;
  if (diff != 0u) {
    const int top = 31 - __builtin_clz(diff);
    theta = (top == 31) ? 0u : (kmax & ~((2u << top) - 1u));
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = theta | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < kSeg; ++i) c += key[i] >= cand ? 1 : 0;
      c = col_sum_i(c);
      if (c >= kk) theta = cand;
    }
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    gt += key[i] > theta ? 1 : 0;
    eq += key[i] == theta ? 1 : 0;
  }
  const int m_eq = kk - col_sum_i(gt);
  int eq_rank = col_exclusive_prefix(eq, g);
  selmask = 0u;
  int nsel = 0;
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    bool s = key[i] > theta;
    if (key[i] == theta) {
      s = eq_rank < m_eq;
      ++eq_rank;
    }
    if (s) {
      selmask |= 1u << i;
      ++nsel;
    }
  }
  TopkResult r;
  r.theta = theta;
  r.nsel_before = col_exclusive_prefix(nsel, g);
  return r;
}

template <typename T, int D, int R>
__global__ __launch_bounds__(256, 2) void select_kernel(const SelectArgs a) {
  typedef SelectSmem<T, D> Smem;
  constexpr int LD = Smem::LD;
  constexpr int KPL = Mfma<T>::KPL;
  constexpr int NF = D / 4 / KPL;              // MFMA steps over d
  constexpr int VE = 16 / (int)sizeof(T);       // elements per 16-byte vector
  constexpr int VPR = D / VE;                   // vectors per landmark row
  constexpr int NV = 64 * VPR / 256;            // staged vectors per thread
  __shared__ Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const uint32_t total = (uint32_t)a.B * a.H * a.N;
  const uint32_t tile = xcd_remap(blockIdx.x, total);
  const int bh = tile / a.N;
  const int c = a.N - 1 - (int)(tile % a.N);   // longest tiles first
  const int b = bh / a.H, h = bh % a.H;
  const int qpos = c * 64 + wave * 16 + m;     // query position of this lane's column
  const int n_cand = c + 1;
  const int n_lt = (n_cand + 63) >> 6;
  const int kk = min(a.k, n_cand);
  const T* Q = static_cast<const T*>(a.q) + (size_t)bh * a.L * D;
  const T* LM = static_cast<const T*>(a.lmk) + (size_t)kv_pair(bh, a.H, a.G) * a.N * D;

  // ---------------- Q-Cal: q~ in the landmark-fragment layout -------------------------------
  typename Mfma<T>::frag qf[NF];
  {
    float qv[D / 4];
#pragma unroll
    for (int eb = 0; eb < D / 16; ++eb) {
      const T* p = Q + (size_t)qpos * D + 16 * eb + 4 * g;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) qv[eb * 4 + rr] = to_f32(p[rr]);
    }
    if (a.r > 0) {
      // delta_q^T[d][query] = W_up[h*D + d][:] . t[query][:]; A = W_up rows, B = t (fp32 split
      // into three bf16 parts on the bf16 path so every product is exact).
      constexpr int KR = Mfma<T>::K;
      constexpr int NRS = 64 / KR;                      // r <= 64
      const int nrs = (a.r + KR - 1) / KR;
      const float* tq = a.tcode + ((size_t)b * a.L + qpos) * a.r;
      const T* WU = static_cast<const T*>(a.w_up) + (size_t)h * D * a.r;
      typename Mfma<T>::frag tb[3][NRS];
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        if (rs < nrs) {
          if constexpr (KPL == 1) {
            const int ai = rs * KR + g;
            tb[0][rs] = ai < a.r ? tq[ai] : 0.f;
          } else {
#pragma unroll
            for (int z = 0; z < KPL; ++z) {
              const int ai = rs * KR + g * KPL + z;
              const float t = ai < a.r ? tq[ai] : 0.f;
              const bf16 t0 = bf16_rne(t);
              const float r1 = t - to_f32(t0);
              const bf16 t1 = bf16_rne(r1);
              const bf16 t2 = bf16_rne(r1 - to_f32(t1));
              tb[0][rs][z] = t0;
              tb[1][rs][z] = t1;
              tb[2][rs][z] = t2;
            }
          }
        }
      }
#pragma unroll
      for (int eb = 0; eb < D / 16; ++eb) {
        f32x4 acc = zero4();
        const T* wrow = WU + (size_t)(eb * 16 + m) * a.r;
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) {
          if (rs < nrs) {
            typename Mfma<T>::frag wa;
            if constexpr (KPL == 1) {
              const int ai = rs * KR + g;
              wa = ai < a.r ? wrow[ai] : 0.f;
              acc = Mfma<T>::mma(wa, tb[0][rs], acc);
            } else {
#pragma unroll
              for (int z = 0; z < KPL; ++z) {
                const int ai = rs * KR + g * KPL + z;
                wa[z] = ai < a.r ? wrow[ai] : bf16_rne(0.f);
              }
              acc = Mfma<T>::mma(wa, tb[0][rs], acc);
              acc = Mfma<T>::mma(wa, tb[1][rs], acc);
              acc = Mfma<T>::mma(wa, tb[2][rs], acc);
            }
          }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) qv[eb * 4 + rr] += acc[rr];
      }
    }
#pragma unroll
    for (int st = 0; st < NF; ++st) {
      if constexpr (KPL == 1) {
        qf[st] = qv[st];
      } else {
#pragma unroll
        for (int z = 0; z < KPL; ++z) qf[st][z] = bf16_rne(qv[st * KPL + z]);
      }
    }
  }

  // ---------------- landmark tile staging ----------------------------------------------------
  u32x4 pre[NV];
  auto load_tile = [&](int lt) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = tid + 256 * u, row = v / VPR, col = v % VPR;
      const int j = lt * 64 + row;
      pre[u] = j < n_cand ? *reinterpret_cast<const u32x4*>(LM + (size_t)j * D + col * VE)
                          : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = tid + 256 * u, row = v / VPR, col = v % VPR;
      *reinterpret_cast<u32x4*>(&sm.lmk[row * LD + col * VE]) = pre[u];
    }
  };
  auto score_tile = [&](int lt, float (&s)[16]) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      f32x4 acc = zero4();
      const T* row = &sm.lmk[(blk * 16 + m) * LD];
#pragma unroll
      for (int st = 0; st < NF; ++st) acc = Mfma<T>::mma(lmk_frag<T>(row, g, st), qf[st], acc);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) s[blk * 4 + rr] = acc[rr];
    }
    if (lt == n_lt - 1) {   // only the last landmark tile holds chunks after the query's own
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (lt * 64 + 16 * (i >> 2) + 4 * g + (i & 3) >= n_cand) s[i] = -INFINITY;
    }
  };

  // ---------------- pass 1: lower bound of the k-th score -----------------------------------
  float tau_thr = -FLT_MAX;
  const bool need_p1 = n_cand > kBufCap;
  if (need_p1) {
    float slot[16 * R];
#pragma unroll
    for (int i = 0; i < 16 * R; ++i) slot[i] = -INFINITY;
    load_tile(0);
    for (int lt = 0; lt < n_lt; ++lt) {
      __syncthreads();
      store_tile();
      __syncthreads();
      if (lt + 1 < n_lt) load_tile(lt + 1);
      float s[16];
      score_tile(lt, s);
      if (R == 2 && (lt & 1)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) slot[16 * (R - 1) + i] = fmaxf(slot[16 * (R - 1) + i], s[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) slot[i] = fmaxf(slot[i], s[i]);
      }
    }
    bitonic_sort_desc<16 * R>(slot);
    const int kq = (a.k + 3) >> 2;
    float thr = slot[0];
#pragma unroll
    for (int i = 1; i < 16 * R; ++i) thr = (i == kq - 1) ? slot[i] : thr;
    tau_thr = col_min(thr);
  }

  // ---------------- pass 2: collect candidates ----------------------------------------------
  float* bs = &sm.bs[(wave * 16 + m) * kBsStride];
  uint16_t* bj = &sm.bj[(wave * 16 + m) * kBjStride];
  int cnt = 0;
  uint32_t key[kSeg];
  int jx[kSeg];
  load_tile(0);
  for (int lt = 0; lt < n_lt; ++lt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (lt + 1 < n_lt) load_tile(lt + 1);
    float s[16];
    score_tile(lt, s);
    uint32_t m16 = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) m16 |= (s[i] >= tau_thr ? 1u : 0u) << i;
    auto spread = [&](uint32_t mm) {
      uint64_t f = 0;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
        f |= (uint64_t)((mm >> (4 * blk)) & 0xFu) << (16 * blk + 4 * g);
      f |= shfl_xor_u64(f, 16);
      f |= shfl_xor_u64(f, 32);
      return f;
    };
    uint64_t full = spread(m16);
    int n_new = __popcll(full);
    if (cnt + n_new > kBufCap) {
      // Cut the buffer to its exact top-k; later chunks must beat the k-th score strictly.
      uint32_t selmask;
      const TopkResult tr = buffer_topk(bs, bj, cnt, a.k, g, key, jx, selmask);
      int pos = tr.nsel_before;
#pragma unroll
      for (int i = 0; i < kSeg; ++i) {
        if (selmask & (1u << i)) {
          bs[pos] = key_f32(key[i]);
          bj[pos] = (uint16_t)jx[i];
          ++pos;
        }
      }
      cnt = a.k;
      tau_thr = key_f32(tr.theta + 1u);
      m16 = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) m16 |= (s[i] >= tau_thr ? 1u : 0u) << i;
      full = spread(m16);
      n_new = __popcll(full);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (m16 & (1u << i)) {
        const int p = 16 * (i >> 2) + 4 * g + (i & 3);
        const int pos = cnt + __popcll(full & ((1ull << p) - 1ull));
        bs[pos] = s[i];
        bj[pos] = (uint16_t)(lt * 64 + p);
      }
    }
    cnt += n_new;
  }

  // ---------------- final top-k and inter-chunk softmax --------------------------------------
  uint32_t selmask;
  const TopkResult tr = buffer_topk(bs, bj, cnt, kk, g, key, jx, selmask);
  uint32_t kmax = 0u;
#pragma unroll
  for (int i = 0; i < kSeg; ++i) kmax = (selmask & (1u << i)) ? max(kmax, key[i]) : kmax;
  const float smax = key_f32(col_max_u(kmax));
  const float zs = a.scale * 1.4426950408889634f;   // scale * log2(e)
  float esum = 0.f;
  float ev[kSeg];
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    ev[i] = (selmask & (1u << i)) ? exp2f((key_f32(key[i]) - smax) * zs) : 0.f;
    esum += ev[i];
  }
  const float inv = 1.f / col_sum(esum);
  const size_t orow = ((size_t)bh * a.L + qpos) * a.k;
  int pos = tr.nsel_before;
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    if (selmask & (1u << i)) {
      a.idx[orow + pos] = jx[i];
      a.w[orow + pos] = ev[i] * inv;
      ++pos;
    }
  }
  for (int p = kk + g; p < a.k; p += 4) {
    a.idx[orow + p] = -1;
    a.w[orow + p] = 0.f;
  }
}

template <typename T, int D>
hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    return launch_select_fast<D>(a, st);   // k <= 64
  }
  const uint32_t total = (uint32_t)a.B * a.H * a.N;
  if (a.k <= 32)
    hipLaunchKernelGGL((select_kernel<T, D, 1>), dim3(total), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((select_kernel<T, D, 2>), dim3(total), dim3(256), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_select<bf16, 64>(const SelectArgs&, hipStream_t);
template hipError_t launch_select<bf16, 128>(const SelectArgs&, hipStream_t);
template hipError_t launch_select<float, 64>(const SelectArgs&, hipStream_t);
template hipError_t launch_select<float, 128>(const SelectArgs&, hipStream_t);

}  // namespace hils
