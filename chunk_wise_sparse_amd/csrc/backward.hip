// Backward pass of the HiLS prefill.
//
// The pages train the chunk selection end to end: the landmark scores are part of the forward
// attention, so the language-modelling loss sends gradients into the landmark keys [HiLS
// Attention explainer (molayo1419.me), "Core idea": gradients reach the landmark
// representations; "HiLS Attention Extrapolates 64x at 90% Retrieval Accuracy": the retrieval
// scores are learned from the loss].  Given dout = dL/do, the gradients are, per row i with
// selection j in sel(i), weights w_j = softmax(s sigma), chunk softmax p_jt over the visible
// keys t of chunk j and o_j = sum_t p_jt v_t:
//   dw_j      = dout . o_j                            (= sum_t p_jt (dout . v_t))
//   dsigma_j  = s w_j (dw_j - sum_j' w_j' dw_j')
//   ds_jt     = w_j p_jt (dout . v_t - dw_j)           (softmax backward of chunk j)
//   dq       += s sum_t ds_jt k_t + sum_j dsigma_j lmk_j   (the second term through q~;
//                                                         its rounding passes gradients)
//   dk_t     += s ds_jt q_i;   dv_t += w_j p_jt dout_i;   dlmk_j += dsigma_j q~_i
//   Q-Cal: dW_up[h] += dq~_i t_i^T, dt_i = sum_h W_up[h]^T dq~_i, dW_down += dt_i h_i^T,
//          dh_i = W_down^T dt_i.
// The top-k choice is a fixed index set (no gradient).  Every (row, chunk) term is local to its
// chunk of 64 keys, so nothing has to be carried between chunks except dsigma's sum.
//
// Kernels (in launch order):
//   bwd_qtilde_kernel     q~ = round(q + W_up t) of every row (Q-Cal only), for dlmk.
//   bwd_row_kernel        row-major: a workgroup takes one chunk's 64 query rows (four 16-row
//                         MFMA blocks) and walks the union of their selections, staging each
//                         chunk's K (two layouts) and V once; per selected (row, chunk) it forms
//                         S^T = K q^T, dP^T = V dout^T, the chunk softmax, dw and ds, and
//                         accumulates dq^T += K^T ds^T; it writes dq (fp32), the chunk's
//                         log-sum-exp and dw per (row, slot), then dsigma per (row, slot).
//   bwd_dqtilde_kernel    dq~ = sum_j dsigma_j lmk_j; dq = dq_attn + dq~ (dq~ kept for Q-Cal).
//   bwd_count/scan/fill   per key/value head: the selections of its query heads inverted into
//                         per-chunk lists of (row, slot), ordered by (head, row) - no atomics
//                         decide the order, so every sum below runs in a fixed order.
//   bwd_chunk_kernel      chunk-major: one workgroup per chunk walks its list in blocks of 16
//                         rows (q, dout, q~ gathered into LDS); wave w owns keys 16w..16w+15
//                         and accumulates dK, dV with MFMA, the chunk's softmax rebuilt from the
//                         saved log-sum-exp; dlmk_j = sum dsigma q~ on the side.
//   bwd_dt / split-K GEMMs / bwd_dh   the Q-Cal factors' gradients, on fp32 MFMA.
#include <float.h>

#include "attn_tiles.h"
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

typedef short short4v __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// q~ for every row (Q-Cal): the same fp32 sum and one rounding to the run dtype as the forward.
// ------------------------------------------------------------------------------------------
// A workgroup takes 64 rows of one (batch, head) (L % 64 == 0): W_up[h] is staged once in LDS
// as fp32 [d][r], thread (row, quarter) holds the row's code t in registers and forms D/4
// elements, each a dot product of length r read from LDS (all rows read the same words).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_qtilde_kernel(const BwdArgs a) {
  constexpr int QD = D / 4;                  // elements per thread
  __shared__ float wl[D * 65];               // W_up[h] rows, stride r + 1 <= 65
  const int tid = threadIdx.x, rl = tid >> 2, qtr = tid & 3;
  const size_t row0 = (size_t)blockIdx.x * 64;          // first row; rows of one (b, h)
  const int bh = (int)(row0 / a.L), h = bh % a.H, b = bh / a.H;
  const int i = (int)(row0 % a.L) + rl;
  const int r = a.r, rs = r + 1;
  const T* wu = static_cast<const T*>(a.w_up) + (size_t)h * D * r;
  for (int x = tid; x < D * r; x += 256) wl[(x / r) * rs + x % r] = to_f32(wu[x]);
  float t[64];
  const float* tp = a.tcode + ((size_t)b * a.L + i) * r;
#pragma unroll
  for (int c = 0; c < 64; ++c) t[c] = c < r ? tp[c] : 0.f;
  __syncthreads();
  const T* q = static_cast<const T*>(a.q) + (row0 + rl) * D + qtr * QD;
  T* qt = static_cast<T*>(a.qt) + (row0 + rl) * D + qtr * QD;
  for (int z = 0; z < QD; ++z) {
    const float* w = wl + (qtr * QD + z) * rs;
    float dq = 0.f;
#pragma unroll
    for (int c = 0; c < 64; ++c)
      if (c < r) dq = fmaf(w[c], t[c], dq);
    qt[z] = from_f32<T>(to_f32(q[z]) + dq);
  }
}

// bf16: the forward selection's own arithmetic, so that q~ is the one the forward scored with.
// One wave per 64 rows of one (batch, head); the offset W_up t by v_mfma_f32_32x32x16_bf16 with t
// split into three bf16 parts (every product exact, fp32 sums in the same order), then one
// rounding of q + offset.  Lane (col, half) holds rows 32 cb + col; MFMA output element e is
// d = 32 db + 8 (e / 4) + 4 half + e % 4.
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <int D, int NRS, bool VEC>
__device__ __forceinline__ void qtilde_rows_mfma(const BwdArgs& a, size_t row0, int b, int h, int i0, int lane) {
  const int col = lane & 31, half = lane >> 5;
  const int r = a.r, nrs = (r + 15) >> 4;
  const bf16* WU = static_cast<const bf16*>(a.w_up) + (size_t)h * D * r;
  const bf16* Q = static_cast<const bf16*>(a.q);
  bf16* QT = static_cast<bf16*>(a.qt);
  auto wfrag = [&](int db, int rs) {           // W_up rows 32 db + col, r-slots 16 rs + 8 half + z
    const bf16* wrow = WU + (size_t)(32 * db + col) * r;
    const int a0 = 16 * rs + 8 * half;
    bf16x8 wa;
    if constexpr (VEC) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(wrow + min(a0, r - 8));
#pragma unroll
      for (int z = 0; z < 8; ++z) wa[z] = a0 < r ? v[z] : bf16_rne(0.f);
    } else {
#pragma unroll
      for (int z = 0; z < 8; ++z) {
        const bf16 v = wrow[min(a0 + z, r - 1)];
        wa[z] = a0 + z < r ? v : bf16_rne(0.f);
      }
    }
    return wa;
  };
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int rq = 32 * cb + col;
    const float* tq = a.tcode + ((size_t)b * a.L + i0 + rq) * r;
    bf16x8 tb[3][NRS];
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
      const int a0 = 16 * rs + 8 * half;
      float tv[8];
      if constexpr (VEC) {
        const float* pt = tq + min(a0, r - 8);
        const f32x4 lo = *reinterpret_cast<const f32x4*>(pt);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(pt + 4);
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          tv[z] = a0 < r ? lo[z] : 0.f;
          tv[4 + z] = a0 < r ? hi[z] : 0.f;
        }
      } else {
#pragma unroll
        for (int z = 0; z < 8; ++z) {
          const float v = tq[min(a0 + z, r - 1)];
          tv[z] = a0 + z < r ? v : 0.f;
        }
      }
#pragma unroll
      for (int z = 0; z < 8; ++z) {
        const float t = tv[z];
        const bf16 t0 = bf16_rne(t);
        const float r1 = t - to_f32(t0);
        const bf16 t1 = bf16_rne(r1);
        tb[0][rs][z] = t0;
        tb[1][rs][z] = t1;
        tb[2][rs][z] = bf16_rne(r1 - to_f32(t1));
      }
    }
    const bf16* qrow = Q + (row0 + rq) * D;
    bf16* orow = QT + (row0 + rq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      bf16x4 qv[4];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) qv[a4] = *reinterpret_cast<const bf16x4*>(qrow + 32 * db + 8 * a4 + 4 * half);
      f32x16 acc = {};
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        if (rs < nrs) {
          const bf16x8 wa = wfrag(db, rs);
#pragma unroll
          for (int p = 0; p < 3; ++p) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, tb[p][rs], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 o;
#pragma unroll
        for (int z = 0; z < 4; ++z) o[z] = bf16_rne(to_f32(qv[a4][z]) + acc[4 * a4 + z]);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * a4 + 4 * half) = o;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_qtilde_mfma_kernel(const BwdArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t row0 = ((size_t)blockIdx.x * 4 + wave) * 64;   // rows of one (b, h): L % 64 == 0
  if (row0 >= (size_t)a.B * a.H * a.L) return;               // wave-uniform
  const int bh = (int)(row0 / a.L), h = bh % a.H, b = bh / a.H, i0 = (int)(row0 % a.L);
  if ((a.r & 7) == 0) {
    if (a.r <= 32) qtilde_rows_mfma<D, 2, true>(a, row0, b, h, i0, lane);
    else qtilde_rows_mfma<D, 4, true>(a, row0, b, h, i0, lane);
  } else {
    if (a.r <= 32) qtilde_rows_mfma<D, 2, false>(a, row0, b, h, i0, lane);
    else qtilde_rows_mfma<D, 4, false>(a, row0, b, h, i0, lane);
  }
}

// ------------------------------------------------------------------------------------------
// Row-major pass.
// ------------------------------------------------------------------------------------------
template <typename T, int D>
struct BwdRowSmem {
  typedef AttnLayout<T, D> Lay;
  alignas(16) char kr[Lay::KBYTES];    // K rows: A operand of S^T
  alignas(16) char kd[Lay::VBYTES];    // K, d-block-major: A operand of dQ^T (transposed reads)
  alignas(16) char vr[Lay::KBYTES];    // V rows: A operand of dP^T
  int nunion;
  uint16_t sidx[64 * 65];
  float sw[64 * 65];
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void bwd_row_kernel(const BwdArgs a) {
  constexpr int NT = 256;
  typedef AttnLayout<T, D> Lay;
  typedef Mfma<T> M;
  constexpr int KPL = M::KPL;
  constexpr int NF = D / 4 / KPL;            // S^T steps over d
  constexpr int NP = 64 / M::K;              // dQ^T steps over the 64 keys
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int NV = 64 * Lay::VPR / NT;     // 16-byte vectors per thread per tensor per chunk
  static_assert(NV >= 1 && (64 * Lay::VPR) % NT == 0, "chunk tile does not split over the threads");
  __shared__ BwdRowSmem<T, D> sm;
  extern __shared__ uint32_t bitmap[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int N = a.L / 64;
  const uint32_t total = (uint32_t)a.B * a.H * N;
  const uint32_t gid = xcd_remap(blockIdx.x, total);
  const int bh = gid / N;
  const int c = N - 1 - (int)(gid % N);      // the group's chunk; longest groups first
  const int q0 = c * 64;
  const int k = a.k, ks = k + 1;
  const int kvp = kv_pair(bh, a.H, a.G);
  const T* Kb = static_cast<const T*>(a.k_in) + (size_t)kvp * a.L * D;
  const T* Vb = static_cast<const T*>(a.v_in) + (size_t)kvp * a.L * D;
  const size_t row0 = (size_t)bh * a.L;

  const int nwords = (c + 1 + 31) >> 5;
  for (int x = tid; x < nwords; x += NT) bitmap[x] = 0u;
  if (tid == 0) sm.nunion = 0;
  for (int r = tid; r < 64; r += NT) sm.sidx[r * ks + k] = (uint16_t)0xFFFF;
  __syncthreads();
  for (int x = tid; x < 64 * k; x += NT) {
    const int r = x / k, e = x - r * k;
    const int j = a.idx[(row0 + q0) * k + x];
    const bool ok = j >= 0 && j <= c;
    sm.sidx[r * ks + e] = ok ? (uint16_t)j : (uint16_t)0xFFFF;
    sm.sw[r * ks + e] = a.w[(row0 + q0) * k + x];
    if (ok) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  {
    int cnt = 0;
    for (int x = tid; x < nwords; x += NT) cnt += __popc(bitmap[x]);
    cnt = (int)wave_sum((float)cnt);
    if (lane == 0) atomicAdd(&sm.nunion, cnt);
  }

  const int rloc = 16 * wave + m, qpos = q0 + rloc;
  const size_t grow = row0 + qpos;
  int ptr = 0;
  typename M::frag qf[NF], df[NF];
  {
    const T* qp = static_cast<const T*>(a.q) + grow * D + g * (D / 4);
    const T* dp = static_cast<const T*>(a.dout) + grow * D + g * (D / 4);
#pragma unroll
    for (int st = 0; st < NF; ++st) {
      qf[st] = load_frag<T>(qp + st * KPL);
      df[st] = load_frag<T>(dp + st * KPL);
    }
  }
  f32x4 acc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc[db] = zero4();
  float dsum = 0.f;                          // sum over the row's chunks of w_j dw_j

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
      const int e = p * VE;
      *reinterpret_cast<u32x4*>(sm.kr + koff(row, e)) = kr[u];
      *reinterpret_cast<u32x4*>(sm.vr + koff(row, e)) = vr[u];
      *reinterpret_cast<u32x4*>(sm.kd + (e >> 4) * Lay::VDB + row * (16 * (int)sizeof(T)) +
                                (e & 15) * (int)sizeof(T)) = kr[u];
    }
  };

  const float zs = a.scale * 1.4426950408889634f;
  auto compute = [&](int j) {
    const int e = rloc * ks + ptr;
    const bool sel = sm.sidx[e] == (uint16_t)j;
    const float wq = sel ? sm.sw[e] : 0.f;
    const int slot = ptr;
    ptr += sel ? 1 : 0;
    if (!__any(sel)) return;
    // S^T and dP^T: lane (m, g) holds row m and keys 16 kb + 4 g + rr.
    float sv[16], pv[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 s4 = zero4(), p4 = zero4();
#pragma unroll
      for (int st = 0; st < NF; ++st) {
        const int off = koff(kb * 16 + m, g * (D / 4) + st * KPL);
        s4 = M::mma(load_frag<T>(reinterpret_cast<const T*>(sm.kr + off)), qf[st], s4);
        p4 = M::mma(load_frag<T>(reinterpret_cast<const T*>(sm.vr + off)), df[st], p4);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        sv[kb * 4 + rr] = s4[rr];
        pv[kb * 4 + rr] = p4[rr];
      }
    }
    if (j == c) {                            // the rows' own chunk: keys after the row masked
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
    mx = col_max(mx) * zs;
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], zs, -mx));
      l += sv[i];
    }
    l = col_sum(l);
    const float inv = 1.0f / l;
    float dw = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] *= inv;                          // p
      dw = fmaf(sv[i], pv[i], dw);
    }
    dw = col_sum(dw);
    if (sel && g == 0) {
      a.lse[grow * k + slot] = mx + __log2f(l);
      a.dw[grow * k + slot] = dw;
    }
    dsum = fmaf(wq, dw, dsum);
    // ds = w p (dP - dw), as the B operand of dQ^T = K^T ds^T.
    typename M::frag sf[NP];
#pragma unroll
    for (int st = 0; st < NP; ++st) {
      if constexpr (KPL == 1) {
        sf[st] = wq * sv[st] * (pv[st] - dw);
      } else {
#pragma unroll
        for (int z = 0; z < KPL; ++z) sf[st][z] = bf16_rne(wq * sv[st * KPL + z] * (pv[st * KPL + z] - dw));
      }
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int st = 0; st < NP; ++st) {
        typename M::frag ka;
        if constexpr (KPL == 1) ka = v_frag_f32<Lay::VDB>(sm.kd, m, g, db, st);
        else ka = v_frag_bf16<Lay::VDB>(sm.kd, m, g, db, st);
        acc[db] = M::mma(ka, sf[st], acc[db]);
      }
  };

  __syncthreads();                           // every wave's union count has landed
  int wi = 0;
  uint32_t cur = bitmap[0];
  auto next_chunk = [&]() -> int {
    while (cur == 0u && wi + 1 < nwords) cur = bitmap[++wi];
    if (cur == 0u) return -1;
    const int j = wi * 32 + __builtin_ctz(cur);
    cur &= cur - 1u;
    return j;
  };
  const int U = sm.nunion;
  int jl = -1;
  auto advance = [&]() -> int {
    const int j = next_chunk();
    if (j >= 0) jl = j;
    return j >= 0 ? j : jl;
  };
  u32x4 kr[NV], vr[NV];
  if (U > 0) {
    int cj = advance();
    load_kv(cj, kr, vr);
    store_kv(kr, vr);
    int cn = advance();
    load_kv(cn, kr, vr);
    __syncthreads();
    for (int t = 0; t < U; ++t) {
      compute(cj);
      __syncthreads();
      store_kv(kr, vr);
      const int cn2 = advance();
      load_kv(cn2, kr, vr);
      __syncthreads();
      cj = cn;
      cn = cn2;
    }
  }

  // dq from the chunk attention (fp32; dq~ is added by the next kernel).  Lane holds d = 16 db +
  // 4 g + rr of its row.
  float* dq = a.dqbuf + grow * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    f32x4 o;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) o[rr] = a.scale * acc[db][rr];
    *reinterpret_cast<f32x4*>(dq + db * 16 + 4 * g) = o;
  }
  // dsigma per slot; the lane that wrote the row's dw reads it back (same thread, in order).
  if (g == 0) {
    const int keff = min(k, c + 1);
    for (int s = 0; s < k; ++s) {
      float ds = 0.f;
      if (s < keff) ds = a.scale * sm.sw[rloc * ks + s] * (a.dw[grow * k + s] - dsum);
      a.dsig[grow * k + s] = ds;
    }
  }
}

// ------------------------------------------------------------------------------------------
// dq~ = sum_j dsigma_j lmk_j per row; dq = dq_attn + dq~ (rounded once); dq~ stays in dqbuf
// for the Q-Cal gradients.
// ------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dqtilde_kernel(const BwdArgs a) {
  constexpr int TPR = D / 8;                 // threads per row, 8 elements each
  constexpr int RPW = 256 / TPR;             // rows per workgroup
  const size_t nrows = (size_t)a.B * a.H * a.L;
  const size_t row = (size_t)blockIdx.x * RPW + threadIdx.x / TPR;
  if (row >= nrows) return;
  const int e0 = (threadIdx.x % TPR) * 8;
  const int bh = (int)(row / a.L);
  const int N = a.L / 64;
  const T* lmk = static_cast<const T*>(a.lmk) + (size_t)kv_pair(bh, a.H, a.G) * N * D + e0;
  const int32_t* ir = a.idx + row * a.k;
  const float* dr = a.dsig + row * a.k;
  float acc[8] = {};
  // Slots in order, eight at a time so that their landmark loads are in flight together; the
  // padding at the end of a row adds exact zeros.
  for (int s0 = 0; s0 < a.k; s0 += 8) {
    int jj[8];
    float ds[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, a.k - 1);
      const int j = ir[s];
      const bool ok = s0 + u < a.k && j >= 0 && j < N;
      jj[u] = ok ? j : 0;
      ds[u] = ok ? dr[s] : 0.f;
    }
    float lv[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const T* lr = lmk + (size_t)jj[u] * D;
      if constexpr (sizeof(T) == 2) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(lr);
#pragma unroll
        for (int z = 0; z < 8; ++z) lv[u][z] = to_f32(x[z]);
      } else {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(lr);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(lr + 4);
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          lv[u][z] = x0[z];
          lv[u][4 + z] = x1[z];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int z = 0; z < 8; ++z) acc[z] = fmaf(ds[u], lv[u][z], acc[z]);
  }
  float* dqb = a.dqbuf + row * D + e0;
  T* dq = static_cast<T*>(a.dq) + row * D + e0;
  const f32x4 q0 = *reinterpret_cast<const f32x4*>(dqb);
  const f32x4 q1 = *reinterpret_cast<const f32x4*>(dqb + 4);
  float sum[8];
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    sum[z] = q0[z] + acc[z];
    sum[4 + z] = q1[z] + acc[4 + z];
  }
  if constexpr (sizeof(T) == 2) {
    bf16x8 o;
#pragma unroll
    for (int z = 0; z < 8; ++z) o[z] = bf16_rne(sum[z]);
    *reinterpret_cast<bf16x8*>(dq) = o;
  } else {
    *reinterpret_cast<f32x4*>(dq) = f32x4{sum[0], sum[1], sum[2], sum[3]};
    *reinterpret_cast<f32x4*>(dq + 4) = f32x4{sum[4], sum[5], sum[6], sum[7]};
  }
  *reinterpret_cast<f32x4*>(dqb) = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<f32x4*>(dqb + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// ------------------------------------------------------------------------------------------
// Per key/value head: the selections of its G query heads as per-chunk lists of
// (g * L + i) << 6 | slot, each list in ascending (g, i) order.  Row blocks of kBwdRB rows over
// the G * L rows: counts per (block, chunk), an exclusive scan down each chunk's column and
// across chunks, then each block fills its rows in order.
// ------------------------------------------------------------------------------------------
constexpr int kBwdRB = 128;

// The G query heads of key/value head bk = b * Hk + hk are consecutive heads, so their G * L
// rows of idx are contiguous; block rblk holds rows rblk * kBwdRB .. of them (fewer in the last).
// Per key/value head bk (blockIdx.y of the list kernels) its slice of the list workspace.
__device__ __forceinline__ int bwd_nrb(const BwdArgs& a) { return (a.G * a.L + kBwdRB - 1) / kBwdRB; }
__device__ __forceinline__ uint32_t* bwd_rbcnt(const BwdArgs& a, int bk) {
  return a.rbcnt + (size_t)bk * bwd_nrb(a) * (a.L / 64);
}
__device__ __forceinline__ uint32_t* bwd_choff(const BwdArgs& a, int bk) {
  return a.choff + (size_t)bk * (a.L / 64 + 1);
}
__device__ __forceinline__ uint32_t* bwd_ent(const BwdArgs& a, int bk) {
  return a.ent + (size_t)bk * a.G * a.L * a.k;
}

__device__ __forceinline__ const int32_t* bwd_idx_rows(const BwdArgs& a, int bk, int rblk) {
  const int Hk = a.H / a.G;
  const int b = bk / Hk, hk = bk % Hk;
  return a.idx + (((size_t)b * a.H + hk * a.G) * a.L + (size_t)rblk * kBwdRB) * a.k;
}
__device__ __forceinline__ int bwd_block_rows(const BwdArgs& a, int rblk) {
  return min(kBwdRB, a.G * a.L - rblk * kBwdRB);
}

__global__ __launch_bounds__(256) void bwd_count_kernel(const BwdArgs a) {
  extern __shared__ uint32_t cnt[];
  const int N = a.L / 64, rblk = blockIdx.x, bk = blockIdx.y;
  for (int j = threadIdx.x; j < N; j += 256) cnt[j] = 0u;
  __syncthreads();
  const int32_t* idx = bwd_idx_rows(a, bk, rblk);
  const int nr = bwd_block_rows(a, rblk);
  for (int x = threadIdx.x; x < nr * a.k; x += 256) {
    const int j = idx[x];
    if (j >= 0 && j < N) atomicAdd(&cnt[j], 1u);
  }
  __syncthreads();
  uint32_t* out = bwd_rbcnt(a, bk) + (size_t)rblk * N;
  for (int j = threadIdx.x; j < N; j += 256) out[j] = cnt[j];
}

// Exclusive prefix down each chunk's column (in place) and the chunk's total.  A workgroup takes
// 16 chunks; 16 threads per chunk sum 16 segments of the column, the segment sums are scanned,
// then each thread rewrites its segment.
__global__ __launch_bounds__(256) void bwd_colscan_kernel(const BwdArgs a) {
  __shared__ uint32_t seg[16][17];
  const int N = a.L / 64, bk = blockIdx.y, nrb = bwd_nrb(a);
  const int jl = threadIdx.x & 15, sg = threadIdx.x >> 4;
  const int j = blockIdx.x * 16 + jl;
  uint32_t* cnt = bwd_rbcnt(a, bk);
  const int per = (nrb + 15) / 16, r0 = min(nrb, sg * per), r1 = min(nrb, r0 + per);
  uint32_t sum = 0;
  if (j < N)
    for (int rb = r0; rb < r1; ++rb) sum += cnt[(size_t)rb * N + j];
  seg[jl][sg] = sum;
  __syncthreads();
  if (sg == 0) {
    uint32_t run = 0;
    for (int t = 0; t < 16; ++t) {
      const uint32_t v = seg[jl][t];
      seg[jl][t] = run;
      run += v;
    }
    if (j < N) bwd_choff(a, bk)[j] = run;     // totals; turned into offsets next
  }
  __syncthreads();
  uint32_t run = seg[jl][sg];
  if (j < N)
    for (int rb = r0; rb < r1; ++rb) {
      const uint32_t v = cnt[(size_t)rb * N + j];
      cnt[(size_t)rb * N + j] = run;
      run += v;
    }
}

__global__ __launch_bounds__(1024) void bwd_offscan_kernel(const BwdArgs a) {
  __shared__ uint32_t part[1024];
  const int N = a.L / 64, t = threadIdx.x;
  uint32_t* choff = bwd_choff(a, blockIdx.x);
  const int per = (N + 1023) / 1024;
  const int b0 = min(N, t * per), e0 = min(N, b0 + per);
  uint32_t s = 0;
  for (int i = b0; i < e0; ++i) s += choff[i];
  part[t] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const uint32_t v = t >= d ? part[t - d] : 0u;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  uint32_t p = part[t] - s;
  for (int i = b0; i < e0; ++i) {
    const uint32_t v = choff[i];
    choff[i] = p;
    p += v;
  }
  if (t == 1023) choff[N] = part[1023];
}

// One wave per row block: the block's selections are staged in LDS, then its rows are appended
// in order (a row's chunks are distinct, so the lanes of one row never share a cursor).
__global__ __launch_bounds__(64) void bwd_fill_kernel(const BwdArgs a) {
  extern __shared__ uint32_t lds[];
  const int N = a.L / 64, rblk = blockIdx.x, bk = blockIdx.y, k = a.k, lane = threadIdx.x;
  const uint32_t* choff = bwd_choff(a, bk);
  const uint32_t* rbcnt = bwd_rbcnt(a, bk);
  uint32_t* ent = bwd_ent(a, bk);
  uint32_t* cur = lds;                       // N cursors
  int32_t* sel = reinterpret_cast<int32_t*>(lds + N);   // kBwdRB * k staged indices
  const int32_t* idx = bwd_idx_rows(a, bk, rblk);
  const int nr = bwd_block_rows(a, rblk);
  for (int j = lane; j < N; j += 64) cur[j] = choff[j] + rbcnt[(size_t)rblk * N + j];
  for (int x = lane; x < nr * k; x += 64) sel[x] = idx[x];
  __syncthreads();
  // One wave: its LDS accesses complete in program order, so row r + 1 reads the cursors row r
  // advanced.
  const uint32_t r0 = (uint32_t)rblk * kBwdRB;
  for (int r = 0; r < nr; ++r) {
    if (lane < k) {
      const int j = sel[r * k + lane];
      if (j >= 0 && j < N) {
        const uint32_t p = cur[j];
        cur[j] = p + 1;
        ent[p] = ((r0 + r) << 6) | (uint32_t)lane;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Chunk-major pass: dK, dV and dlmk of one chunk of key/value head bk per workgroup.
// ------------------------------------------------------------------------------------------
constexpr int kBwdBR = 32;                   // list entries (rows) per block of the chunk pass

template <typename T, int D>
struct BwdChunkSmem {
  static constexpr int RB = 16 * (int)sizeof(T);      // bytes of one row within a d-block
  static constexpr int DBS = kBwdBR * RB + 32;         // d-block stride: the block's rows + pad
  alignas(16) char qs[(D / 16) * DBS];                 // gathered q rows, d-block-major
  alignas(16) char ds[(D / 16) * DBS];                 // gathered dout rows
  alignas(16) char ts[(D / 16) * DBS];                 // gathered q~ rows
  float rw[kBwdBR], rlse[kBwdBR], rdw[kBwdBR], rsig[kBwdBR];
  int rpos[kBwdBR];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_chunk_kernel(const BwdArgs a) {
  typedef BwdChunkSmem<T, D> S;
  typedef Mfma<T> M;
  constexpr int KPL = M::KPL;
  constexpr int NF = D / 4 / KPL;            // S steps over d
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int VPR = D / VE;                // 16-byte vectors per row
  __shared__ S sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int N = a.L / 64, j = blockIdx.x, bk = blockIdx.y;
  const int Hk = a.H / a.G, b = bk / Hk, hk = bk % Hk;
  const uint32_t* ent = bwd_ent(a, bk);
  const size_t kvoff = (size_t)bk * a.L * D;
  const int key = 16 * wave + n;             // this lane's key within the chunk (B operands)
  const int kpos = j * 64 + key;
  const T* krow = static_cast<const T*>(a.k_in) + kvoff + (size_t)kpos * D + g * (D / 4);
  const T* vrow = static_cast<const T*>(a.v_in) + kvoff + (size_t)kpos * D + g * (D / 4);
  typename M::frag kf[NF], vf[NF];
#pragma unroll
  for (int st = 0; st < NF; ++st) {
    kf[st] = load_frag<T>(krow + st * KPL);
    vf[st] = load_frag<T>(vrow + st * KPL);
  }
  f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) dk[db] = dv[db] = zero4();
  float dl = 0.f;                            // dlmk, dim wave * D/4 + lane (lanes < D/4)
  const float zs = a.scale * 1.4426950408889634f;
  const T* qt_base = static_cast<const T*>(a.r > 0 ? a.qt : a.q);

  const uint32_t e0 = bwd_choff(a, bk)[j], e1 = bwd_choff(a, bk)[j + 1];
  // The next block's rows and per-row values are loaded into registers while the current block
  // is computed, and the list entries that address them one block earlier still, so that no
  // load waits on an entry load issued in the same step (the vector memory counter completes
  // in order: such a wait would also drain the loads in flight).  Loads are unconditional:
  // entries past the list end re-read its last entry, and their per-row values are replaced by
  // inert ones (w = 0, no position) only when the block is put into LDS.
  constexpr int NGV = kBwdBR * VPR / 256;   // 16-byte vectors per thread per tensor
  static_assert(NGV >= 1 && kBwdBR * VPR == 256 * NGV, "gather tile does not split over the threads");
  u32x4 gq[NGV], gd[NGV], gt[NGV];
  uint32_t en_v[NGV], en_s;                  // entries of the block after the next
  bool ok_s = false, ok_n = false;
  float g_w = 0.f, g_lse = INFINITY, g_dw = 0.f, g_sg = 0.f;
  int g_pos = -1;
  auto fetch_ent = [&](uint32_t base) {
#pragma unroll
    for (int u = 0; u < NGV; ++u) en_v[u] = ent[min(base + (uint32_t)((tid + 256 * u) / VPR), e1 - 1u)];
    const uint32_t x = base + (uint32_t)(tid % kBwdBR);
    en_s = ent[min(x, e1 - 1u)];
    ok_s = x < e1;
  };
  auto fetch = [&]() {                       // from the entries in en_v / en_s
#pragma unroll
    for (int u = 0; u < NGV; ++u) {
      const int p = (tid + 256 * u) % VPR;
      const uint32_t en = en_v[u];
      const int gi = (int)(en >> 6), gq_ = gi / a.L, i = gi % a.L;
      const size_t row = ((size_t)b * a.H + hk * a.G + gq_) * a.L + i;
      gq[u] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.q) + row * D + p * VE);
      gd[u] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dout) + row * D + p * VE);
      gt[u] = *reinterpret_cast<const u32x4*>(qt_base + row * D + p * VE);
    }
    const uint32_t en = en_s;
    const int slot = (int)(en & 63u), gi = (int)(en >> 6), gq_ = gi / a.L, i = gi % a.L;
    const size_t rs = (((size_t)b * a.H + hk * a.G + gq_) * a.L + i) * a.k + slot;
    g_w = a.w[rs];
    g_lse = a.lse[rs];
    g_dw = a.dw[rs];
    g_sg = a.dsig[rs];
    g_pos = i;
    ok_n = ok_s;
  };
  auto put = [&]() {
#pragma unroll
    for (int u = 0; u < NGV; ++u) {
      const int v = tid + 256 * u;
      const int r = v / VPR, p = v % VPR, e = p * VE;
      const int off = (e >> 4) * S::DBS + r * S::RB + (e & 15) * (int)sizeof(T);
      *reinterpret_cast<u32x4*>(sm.qs + off) = gq[u];
      *reinterpret_cast<u32x4*>(sm.ds + off) = gd[u];
      *reinterpret_cast<u32x4*>(sm.ts + off) = gt[u];
    }
    if (tid < kBwdBR) {
      sm.rw[tid] = ok_n ? g_w : 0.f;
      sm.rlse[tid] = ok_n ? g_lse : INFINITY;
      sm.rdw[tid] = ok_n ? g_dw : 0.f;
      sm.rsig[tid] = ok_n ? g_sg : 0.f;
      sm.rpos[tid] = ok_n ? g_pos : -1;
    }
  };
  if (e0 < e1) {
    fetch_ent(e0);
    fetch();
    fetch_ent(e0 + kBwdBR);
  }
  for (uint32_t base = e0; base < e1; base += kBwdBR) {
    put();
    __syncthreads();
    fetch();                                 // the next block (inert past the list end)
    fetch_ent(base + 2 * kBwdBR);
    // S[q][key] = Q K^T and dP[q][key] = dout V^T for the block's two 16-row tiles: lane (n, g)
    // holds key n of the wave and rows q = 16 t + 4 g + rr.
    float pw[2][4], dsv[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 s4 = zero4(), p4 = zero4();
#pragma unroll
      for (int st = 0; st < NF; ++st) {
        const int e = g * (D / 4) + st * KPL;
        const int off = (e >> 4) * S::DBS + (16 * t + n) * S::RB + (e & 15) * (int)sizeof(T);
        s4 = M::mma(load_frag<T>(reinterpret_cast<const T*>(sm.qs + off)), kf[st], s4);
        p4 = M::mma(load_frag<T>(reinterpret_cast<const T*>(sm.ds + off)), vf[st], p4);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int q = 16 * t + 4 * g + rr;
        const int pos = sm.rpos[q];
        float p = __builtin_amdgcn_exp2f(fmaf(s4[rr], zs, -sm.rlse[q]));
        if (pos < kpos) p = 0.f;             // the key lies after the row (or no row)
        const float w = sm.rw[q];
        pw[t][rr] = w * p;
        dsv[t][rr] = w * p * (p4[rr] - sm.rdw[q]);
      }
    }
    // dV[key][e] += sum_q (w p)[q][key] dout[q][e];  dK[key][e] += sum_q ds[q][key] q[q][e]:
    // MFMA with the block's 32 rows as the contraction, contraction slot (g, z) being row
    // 16 (z / 4) + 4 g + z % 4 in A = (w p)^T / ds^T (lane (n, g): key n) and in B = the row
    // tiles (column e, read transposed).
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      if constexpr (KPL == 1) {
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int off = db * S::DBS + (16 * (st >> 2) + 4 * g + (st & 3)) * S::RB + n * 4;
          const float dov = *reinterpret_cast<const float*>(sm.ds + off);
          const float qv = *reinterpret_cast<const float*>(sm.qs + off);
          dv[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(pw[st >> 2][st & 3], dov, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(dsv[st >> 2][st & 3], qv, dk[db], 0, 0, 0);
        }
      } else {
        // lane (n, g) gets column n of rows 4 g..4 g + 3 (and 16 + those) of d-block db
        const int off = db * S::DBS + (4 * g + (n >> 2)) * S::RB + 8 * (n & 3);
        const short4v d0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(void*)(sm.ds + off));
        const short4v d1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(void*)(sm.ds + off + 16 * S::RB));
        const short4v q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(void*)(sm.qs + off));
        const short4v q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(void*)(sm.qs + off + 16 * S::RB));
        bf16x8 pa, sa;
#pragma unroll
        for (int z = 0; z < 8; ++z) {
          pa[z] = bf16_rne(pw[z >> 2][z & 3]);
          sa[z] = bf16_rne(dsv[z >> 2][z & 3]);
        }
        const bf16x4 d0b = __builtin_bit_cast(bf16x4, d0), d1b = __builtin_bit_cast(bf16x4, d1);
        const bf16x4 q0b = __builtin_bit_cast(bf16x4, q0), q1b = __builtin_bit_cast(bf16x4, q1);
        dv[db] = Mfma<bf16>::mma(pa, __builtin_shufflevector(d0b, d1b, 0, 1, 2, 3, 4, 5, 6, 7), dv[db]);
        dk[db] = Mfma<bf16>::mma(sa, __builtin_shufflevector(q0b, q1b, 0, 1, 2, 3, 4, 5, 6, 7), dk[db]);
      }
    }
    // dlmk: dims wave * D/4 + lane, summed over the block's rows in order.
    if (lane < D / 4) {
      const int e = wave * (D / 4) + lane;
#pragma unroll
      for (int q = 0; q < kBwdBR; ++q) {
        const T tv = *reinterpret_cast<const T*>(sm.ts + (e >> 4) * S::DBS + q * S::RB + (e & 15) * (int)sizeof(T));
        dl = fmaf(sm.rsig[q], to_f32(tv), dl);
      }
    }
    __syncthreads();
  }
  // outputs: lane (n, g) holds rows (keys) 16 wave + 4 g + rr, column e = 16 db + n
  T* dko = static_cast<T*>(a.dk) + kvoff + (size_t)j * 64 * D;
  T* dvo = static_cast<T*>(a.dv) + kvoff + (size_t)j * 64 * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const size_t o = (size_t)(16 * wave + 4 * g + rr) * D + 16 * db + n;
      dko[o] = from_f32<T>(a.scale * dk[db][rr]);
      dvo[o] = from_f32<T>(dv[db][rr]);
    }
  if (lane < D / 4)
    static_cast<T*>(a.dlmk)[((size_t)bk * N + j) * D + wave * (D / 4) + lane] = from_f32<T>(dl);
}

// ------------------------------------------------------------------------------------------
// Q-Cal gradients.  tok = b * L + i indexes the B * L tokens.  The products run on fp32 MFMA
// (v_mfma_f32_32x32x2_f32): A lane (i, h) holds row i and contraction slot h, B lane (j, h) holds
// slot h and column j, and output element e of lane (j, h) is row 8 (e / 4) + 4 h + e % 4,
// column j.  Which contraction index a slot stands for at a step is free as long as A and B
// agree; each kernel picks it so that a lane's operands come from one vector load.  NCB is the
// number of 32-code blocks (r <= 32 * NCB).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_f32(float x, float y, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, c, 0, 0, 0);
}

// dt[tok][c] = sum_x dq~[tok][x] W_up[x][c], x = h d + e.  A wave takes 32 tokens and every code;
// the workgroup's four waves share slices of W_up^T (128 x) staged in LDS as fp32.  In a 32-x
// step group, step s pairs x = x1 + s (slot 0) with x1 + 16 + s (slot 1): lane (token, h) reads
// its 16 values of dq~ as four 16-byte loads (d % 16 == 0: they stay inside one head).
template <typename T, int NCB>
__global__ __launch_bounds__(256) void bwd_dt_kernel(const BwdArgs a) {
  constexpr int XB = 128, NC = 32 * NCB, WS = XB + 4;
  __shared__ float wt[NC * WS];                // W_up^T slice: [code][x]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int ntok = a.B * a.L, HD = a.H * a.d;
  const int tb = (blockIdx.x * 4 + wave) * 32;
  const int tok = tb + li;
  const bool tv = tok < ntok;
  const int b = tv ? tok / a.L : 0, i = tv ? tok % a.L : 0;
  const T* wu = static_cast<const T*>(a.w_up);
  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  for (int x0 = 0; x0 < HD; x0 += XB) {
    __syncthreads();
    for (int v = tid; v < XB * NC; v += 256) {
      const int xr = v / NC, c = v % NC;
      wt[c * WS + xr] = (c < a.r && x0 + xr < HD) ? to_f32(wu[(size_t)(x0 + xr) * a.r + c]) : 0.f;
    }
    __syncthreads();
#pragma unroll 2
    for (int xs = 0; xs < XB; xs += 32) {
      const int x = x0 + xs + 16 * lh;
      f32x4 xv[4];
      if (tv && x < HD) {
        const float* src = a.dqbuf + (((size_t)b * a.H + x / a.d) * a.L + i) * a.d + x % a.d;
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[u] = *reinterpret_cast<const f32x4*>(src + 4 * u);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float* wr = wt + (32 * cb + li) * WS + xs + 16 * lh;
        f32x4 wv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) wv[u] = *reinterpret_cast<const f32x4*>(wr + 4 * u);
#pragma unroll
        for (int st = 0; st < 16; ++st) acc[cb] = mfma_f32(xv[st >> 2][st & 3], wv[st >> 2][st & 3], acc[cb]);
      }
    }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int c = 32 * cb + li;
    if (c < a.r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = tb + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (t < ntok) a.dt[(size_t)t * a.r + c] = acc[cb][e];
      }
    }
  }
}

// Split-K outer-product sums over tokens: part[s][x][c] = sum over the tokens of split s of
// X[tok][x] Y[tok][c], Y = [tokens, r] fp32.  kind 0: X = dq~ (x over H d), Y = t (for dW_up);
// kind 1: X = h (x over the hidden size), Y = dt (for dW_down).  A wave takes 128 x as four
// 32-row output blocks, lane i of block q standing for x = xw + 4 i + q (one vector load of four
// x per lane and token), and every code; step u pairs tokens t0 + 2 u (slot 0) and t0 + 2 u + 1
// (slot 1).  The tokens of a split are summed in order.
template <typename T, int KIND, int NCB>
__global__ __launch_bounds__(256) void bwd_splitk_kernel(const BwdArgs a, int X, int tok_per_split) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int ntok = a.B * a.L, s = blockIdx.y;
  const int t_begin = s * tok_per_split, t_end = min(ntok, t_begin + tok_per_split);
  const int xw = (blockIdx.x * 4 + wave) * 128;
  if (xw >= X) return;                         // wave-uniform; X % 128 == 0 or the tail is masked
  const int x = xw + 4 * li;
  const bool xok = x < X;
  const int xc = xok ? x : 0;                  // a valid address for the masked lanes
  const float* Y = KIND == 0 ? a.tcode : a.dt;
  int cy[NCB];
  bool cok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    cok[cb] = 32 * cb + li < a.r;
    cy[cb] = cok[cb] ? 32 * cb + li : 0;
  }
  auto load_x = [&](int tok) -> f32x4 {
    f32x4 v;
    if constexpr (KIND == 0) {
      const int b = tok / a.L, i = tok % a.L;
      v = *reinterpret_cast<const f32x4*>(a.dqbuf + (((size_t)b * a.H + xc / a.d) * a.L + i) * a.d + xc % a.d);
    } else if constexpr (sizeof(T) == 2) {
      const bf16x4 hv = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(a.h) + (size_t)tok * a.Dh + xc);
#pragma unroll
      for (int z = 0; z < 4; ++z) v[z] = to_f32(hv[z]);
    } else {
      v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.h) + (size_t)tok * a.Dh + xc);
    }
    return xok ? v : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  f32x16 acc[4][NCB];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[q][cb] = f32x16{};
  constexpr int U = 8;                         // token pairs per unrolled step group
  int t0 = t_begin;
  for (; t0 + 2 * U <= t_end; t0 += 2 * U) {
    f32x4 xa[U];
    float yb[U][NCB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tok = t0 + 2 * u + lh;
      xa[u] = load_x(tok);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float y = Y[(size_t)tok * a.r + cy[cb]];
        yb[u][cb] = cok[cb] ? y : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[q][cb] = mfma_f32(xa[u][q], yb[u][cb], acc[q][cb]);
  }
  for (; t0 < t_end; t0 += 2) {
    const int tok = t0 + lh;
    const bool ok = tok < t_end;
    const f32x4 xv = load_x(ok ? tok : t0);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float y = Y[(size_t)(ok ? tok : t0) * a.r + cy[cb]];
      const float yv = ok && cok[cb] ? y : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q][cb] = mfma_f32(ok ? xv[q] : 0.f, yv, acc[q][cb]);
    }
  }
  // lane (c, h), element e: x = xw + 4 (8 (e / 4) + 4 h + e % 4) + q
  float* part = a.gpart + (size_t)s * X * 64;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int xo = xw + 4 * (8 * (e >> 2) + 4 * lh + (e & 3)) + q;
        if (xo < X) part[(size_t)xo * 64 + 32 * cb + li] = acc[q][cb][e];
      }
}

// out = sum of the splits in order.  kind 0: out[x][c] ([H*d, r]); kind 1: out[c][x] ([r, hidden]).
template <typename T, int KIND>
__global__ __launch_bounds__(256) void bwd_splitk_reduce_kernel(const BwdArgs a, int X, int splits, void* out) {
  const size_t n = (size_t)X * a.r;
  for (size_t v = (size_t)blockIdx.x * 256 + threadIdx.x; v < n; v += (size_t)gridDim.x * 256) {
    int x, c;
    if constexpr (KIND == 0) {
      x = (int)(v / a.r);
      c = (int)(v % a.r);
    } else {
      c = (int)(v / X);
      x = (int)(v % X);
    }
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += a.gpart[((size_t)sp * X + x) * 64 + c];
    static_cast<T*>(out)[v] = from_f32<T>(s);
  }
}

// dh[tok][x] = sum_c dt[tok][c] W_down[c][x].  A wave takes 32 tokens and 512 hidden columns in
// four passes of 128 (four 32-column output blocks, lane j of block q standing for x = x1 + 4 j +
// q); step st pairs codes st (slot 0) and 16 NCB + st (slot 1).  The tokens' codes are loaded
// once; W_down is read in 8- or 16-byte pieces (four x per lane and code).
template <typename T, int NCB>
__global__ __launch_bounds__(256) void bwd_dh_kernel(const BwdArgs a) {
  constexpr int NS = 16 * NCB;                 // steps over the codes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int ntok = a.B * a.L;
  const int tb = blockIdx.x * 32;
  const int xw = (blockIdx.y * 4 + wave) * 512;
  if (xw >= a.Dh) return;                      // wave-uniform
  const T* wd = static_cast<const T*>(a.w_down);
  float ta[NS];
  {
    const int tok = min(tb + li, ntok - 1);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int c = NS * lh + st;
      const float v = a.dt[(size_t)tok * a.r + min(c, a.r - 1)];
      ta[st] = c < a.r ? v : 0.f;
    }
  }
  for (int x1 = xw; x1 < min(a.Dh, xw + 512); x1 += 128) {
    f32x16 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int c = NS * lh + st;
      float wv[4];
      const T* src = wd + (size_t)min(c, a.r - 1) * a.Dh + x1 + 4 * li;
      if constexpr (sizeof(T) == 2) {
        const bf16x4 w4 = *reinterpret_cast<const bf16x4*>(src);
#pragma unroll
        for (int z = 0; z < 4; ++z) wv[z] = to_f32(w4[z]);
      } else {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
        for (int z = 0; z < 4; ++z) wv[z] = w4[z];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = mfma_f32(ta[st], c < a.r ? wv[q] : 0.f, acc[q]);
    }
    // lane (j, h), element e: token tb + 8 (e / 4) + 4 h + e % 4, x = x1 + 4 j + q
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tb + 8 * (e >> 2) + 4 * lh + (e & 3);
      if (t < ntok) {
        T* dst = static_cast<T*>(a.dh) + (size_t)t * a.Dh + x1 + 4 * li;
        if constexpr (sizeof(T) == 2) {
          bf16x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = bf16_rne(acc[q][e]);
          *reinterpret_cast<bf16x4*>(dst) = o;
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0][e], acc[1][e], acc[2][e], acc[3][e]};
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Launcher.
// ------------------------------------------------------------------------------------------
size_t bwd_rbcnt_words(int G, int L, int N) { return (size_t)((G * L + kBwdRB - 1) / kBwdRB) * N; }   // per head
int bwd_splits(int ntok) { return max(1, min(256, ntok / 1024)); }

template <typename T, int NCB>
void launch_qcal_grads(const BwdArgs& a, hipStream_t st) {
  const int ntok = a.B * a.L;
  hipLaunchKernelGGL((bwd_dt_kernel<T, NCB>), dim3((ntok + 127) / 128), dim3(256), 0, st, a);
  const int S = bwd_splits(ntok), per = (ntok + S - 1) / S;
  const int HD = a.H * a.d;
  hipLaunchKernelGGL((bwd_splitk_kernel<T, 0, NCB>), dim3((HD + 511) / 512, S), dim3(256), 0, st, a, HD, per);
  hipLaunchKernelGGL((bwd_splitk_reduce_kernel<T, 0>), dim3(1024), dim3(256), 0, st, a, HD, S, a.dw_up);
  hipLaunchKernelGGL((bwd_splitk_kernel<T, 1, NCB>), dim3((a.Dh + 511) / 512, S), dim3(256), 0, st, a, a.Dh, per);
  hipLaunchKernelGGL((bwd_splitk_reduce_kernel<T, 1>), dim3(1024), dim3(256), 0, st, a, a.Dh, S, a.dw_down);
  hipLaunchKernelGGL((bwd_dh_kernel<T, NCB>), dim3((ntok + 31) / 32, (a.Dh + 2047) / 2048), dim3(256), 0, st, a);
}

template <typename T, int D>
hipError_t launch_prefill_bwd(const BwdArgs& a, hipStream_t st) {
  const int N = a.L / 64, ntok = a.B * a.L;
  if (a.r > 0) {
    const size_t tiles = (size_t)a.B * a.H * a.L / 64;
    if constexpr (sizeof(T) == 2)
      hipLaunchKernelGGL((bwd_qtilde_mfma_kernel<D>), dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_qtilde_kernel<T, D>), dim3((unsigned)tiles), dim3(256), 0, st, a);
  }
  const size_t bm = (size_t)((N + 31) / 32) * 4;
  hipLaunchKernelGGL((bwd_row_kernel<T, D>), dim3((uint32_t)a.B * a.H * N), dim3(256), bm, st, a);
  constexpr int RPW = 256 / (D / 8);
  const size_t nrows = (size_t)a.B * a.H * a.L;
  hipLaunchKernelGGL((bwd_dqtilde_kernel<T, D>), dim3((unsigned)((nrows + RPW - 1) / RPW)), dim3(256), 0, st, a);
  const int nrb = (a.G * a.L + kBwdRB - 1) / kBwdRB;
  const int nkv = a.B * (a.H / a.G);        // every key/value head at once (blockIdx.y)
  hipLaunchKernelGGL(bwd_count_kernel, dim3(nrb, nkv), dim3(256), (size_t)N * 4, st, a);
  hipLaunchKernelGGL(bwd_colscan_kernel, dim3((N + 15) / 16, nkv), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_offscan_kernel, dim3(nkv), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(bwd_fill_kernel, dim3(nrb, nkv), dim3(64), (size_t)(N + kBwdRB * a.k) * 4, st, a);
  hipLaunchKernelGGL((bwd_chunk_kernel<T, D>), dim3(N, nkv), dim3(256), 0, st, a);
  if (a.r > 0) {
    if (a.r <= 32) launch_qcal_grads<T, 1>(a, st);
    else launch_qcal_grads<T, 2>(a, st);
  }
  return hipGetLastError();
}

template hipError_t launch_prefill_bwd<bf16, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_prefill_bwd<bf16, 128>(const BwdArgs&, hipStream_t);
template hipError_t launch_prefill_bwd<float, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_prefill_bwd<float, 128>(const BwdArgs&, hipStream_t);

}  // namespace hils
