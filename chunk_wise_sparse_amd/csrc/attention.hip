// Intra-chunk attention and fusion for prefill.
//
// Method: [HiLS Attention explainer (molayo1419.me), "Core idea", level 2] ordinary softmax
// attention over the tokens of each selected chunk; ["HiLS Attention Extrapolates 64x at 90%
// Retrieval Accuracy"] each chunk is attended independently and the per-chunk outputs are summed
// with the inter-chunk weights.  Because every chunk's softmax is normalised on its own, the
// fused output is sum_j (w_j / l_j) * sum_t exp(a_t - m_j) v_t: no rescaling across chunks.
//
// Kernels (the pages' "load the union once" idea, designed afresh for wave64/MFMA): a workgroup
// takes consecutive queries of one (batch, head) - several 64-query chunks - and walks the union
// of their selected chunks in ascending order.  Each union chunk's K and V are staged once in
// LDS and shared by all waves.
//   chunk_attention_block_kernel (bf16, k <= 32) and chunk_attention_block64_kernel (bf16,
//     k <= 64): 128 queries, eight waves of one 16-row MFMA block each; a wave computes the
//     chunks its 16 rows selected.
//   chunk_attention_kernel (fp32, or sequences not a multiple of 128): wave w owns rows
//     32w..32w+31 as two 16-row blocks
//     and skips a chunk that none of its 32 rows selected; otherwise both blocks run
//     (branch-free, so the two blocks' MFMA and softmax work interleave).
// Rows of a block that did not select the chunk get weight 0.
//   S^T[key][q] = K . Q^T  : A = K rows (LDS), B = raw q (registers);
//                            lane (m, g) holds query m and keys 16*kb + 4g + rr;
//   O^T[d][q] += V^T . P'^T: A = V^T via LDS transpose reads, B = P' = p * (w_j / l_j).
// K and V are loaded into registers and then written to LDS.  The one-block kernels keep one LDS
// stage and the next chunk in registers (two barriers per chunk); the two-block kernel computes
// chunk t from one of two stages while chunk t+1 is written to the other and chunk t+2 is in
// flight.
//
// Chunk-major mode (cm_* kernels, bf16, chosen by the caller): for selections whose rows share
// few chunks, one (batch, head) pair at a time is turned into per-chunk row lists, each chunk's
// K/V is staged once per 128 rows that chose it, and every row sums its per-slot partial outputs
// in slot order.
#include <float.h>

#include "attn_tiles.h"
#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

// Selection of the group's rows, staged once: chunk index (u16, 0xFFFF = padding) and weight.
// The union bitmap, one bit per chunk of the sequence, is the dynamic part of LDS.
template <typename T, int D, int QG, int KMAX, int STAGES>
struct AttnSmem {
  typedef float WT;
  alignas(16) char k[STAGES][AttnLayout<T, D>::KBYTES];
  alignas(16) char v[STAGES][AttnLayout<T, D>::VBYTES];
  int nunion;
  uint16_t sidx[QG * (KMAX + 1)];
  WT sw[QG * (KMAX + 1)];
};

template <typename T, int D, int NW, int KMAX, int STAGES>
__global__ __launch_bounds__(NW * 64, 1) void chunk_attention_kernel(const AttnArgs a) {
  static_assert(STAGES == 1 || STAGES == 2, "one or two LDS stages");
  constexpr int QG = 32 * NW;                // queries per workgroup
  typedef AttnSmem<T, D, QG, KMAX, STAGES> Smem;
  typedef AttnLayout<T, D> Lay;
  constexpr int KPL = Mfma<T>::KPL;
  constexpr int NF = D / 4 / KPL;            // QK^T steps over d
  // The chunk's V fragments stay in registers between the two blocks' PV (64 VGPRs at d = 128).
  constexpr bool kSplitPV = true;
  constexpr int NP = 64 / Mfma<T>::K;        // PV steps over the 64 keys
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int NT = NW * 64;                // threads
  constexpr int NV = 64 * Lay::VPR / NT;     // 16-byte vectors per thread per tensor per chunk
  static_assert(NV >= 1 && (64 * Lay::VPR) % NT == 0, "chunk tile does not split over the threads");
  __shared__ Smem sm;
  extern __shared__ uint32_t bitmap[];       // ceil(N / 32) words

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int groups = a.L / QG;
  const uint32_t total = (uint32_t)a.B * a.H * groups;
  const uint32_t gid = xcd_remap(blockIdx.x, total);
  const int bh = gid / groups;
  const int q0 = (int)(gid % groups) * QG;   // first query position of the group
  const int c_last = (q0 + QG - 1) >> 6;     // last chunk a row of the group may select
  const int k = a.topk;
  const int ks = k + 1;                      // staged row stride (odd: rows hit distinct banks)
  const T* Kb = static_cast<const T*>(a.key) + (size_t)kv_pair(bh, a.H, a.G) * a.L * D;
  const T* Vb = static_cast<const T*>(a.val) + (size_t)kv_pair(bh, a.H, a.G) * a.L * D;
  const int32_t* bt = a.block_table ? a.block_table + (size_t)(bh / a.H) * a.bt_stride : nullptr;
  const int kvh = (bh % a.H) / a.G;
  const size_t row0 = (size_t)bh * a.L;

  // Stage the group's selections and build the union bitmap (causal chunks only).
  const int nwords = (c_last + 1 + 31) >> 5;
  for (int x = tid; x < nwords; x += NT) bitmap[x] = 0u;
  if (tid == 0) sm.nunion = 0;
  for (int r = tid; r < QG; r += NT) sm.sidx[r * ks + k] = (uint16_t)0xFFFF;   // end sentinel
  __syncthreads();
  for (int x = tid; x < QG * k; x += NT) {
    const int r = x / k, e = x - r * k;
    const int j = a.idx[(row0 + q0) * k + x];
    const bool ok = j >= 0 && j <= c_last;
    sm.sidx[r * ks + e] = ok ? (uint16_t)j : (uint16_t)0xFFFF;
    sm.sw[r * ks + e] = static_cast<typename Smem::WT>(a.w[(row0 + q0) * k + x]);
    if (ok) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  {
    int cnt = 0;
    for (int x = tid; x < nwords; x += NT) cnt += __popc(bitmap[x]);
    cnt = (int)wave_sum((float)cnt);   // exact: at most 65536
    if (lane == 0) atomicAdd(&sm.nunion, cnt);
  }

  // This lane's rows: block b covers rows 32*wave + 16*b + m of the group.
  int qpos[2], crow[2], rloc[2], ptr[2];
  typename Mfma<T>::frag qf[2][NF];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    rloc[b] = 32 * wave + 16 * b + m;
    qpos[b] = q0 + rloc[b];
    crow[b] = qpos[b] >> 6;
    ptr[b] = 0;
    const T* qp = static_cast<const T*>(a.q) + (row0 + qpos[b]) * D + g * (D / 4);
#pragma unroll
    for (int st = 0; st < NF; ++st) qf[b][st] = load_frag<T>(qp + st * KPL);
  }
  // Wait for q here, once, rather than let the loop's first use carry an unknown load count.
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int st = 0; st < NF; ++st) asm volatile("" ::"v"(qf[b][st]));
  f32x4 acc_o[2][D / 16];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc_o[b][db] = zero4();

  // Thread -> 16-byte vector u of a chunk: row v / VPR, vector v % VPR (consecutive threads
  // read consecutive bytes of K and of V).
  auto load_kv = [&](int j, u32x4 (&kr)[NV], u32x4 (&vr)[NV]) {
    const T* kc = kv_chunk<T, D>(Kb, static_cast<const T*>(a.key), bt, a.num_pages, a.H / a.G, kvh, j);
    const T* vc = kv_chunk<T, D>(Vb, static_cast<const T*>(a.val), bt, a.num_pages, a.H / a.G, kvh, j);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = tid + NT * u;
      kr[u] = *reinterpret_cast<const u32x4*>(kc + (size_t)v * VE);
      vr[u] = *reinterpret_cast<const u32x4*>(vc + (size_t)v * VE);
    }
  };
  auto store_kv = [&](int stg, const u32x4 (&kr)[NV], const u32x4 (&vr)[NV]) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = tid + NT * u;
      const int row = v / Lay::VPR, p = v % Lay::VPR;
      *reinterpret_cast<u32x4*>(sm.k[stg] + row * Lay::KLD + p * 16) = kr[u];
      const int e = p * VE;                  // first element of the vector
      *reinterpret_cast<u32x4*>(sm.v[stg] + (e >> 4) * Lay::VDB + row * (16 * (int)sizeof(T)) +
                                (e & 15) * (int)sizeof(T)) = vr[u];
    }
  };

  __syncthreads();
  // Union iterator, identical in every thread: ascending chunk order.
  int wi = 0;
  uint32_t cur = bitmap[0];
  auto next_chunk = [&]() -> int {
    while (cur == 0u && wi + 1 < nwords) cur = bitmap[++wi];
    if (cur == 0u) return -1;
    const int j = wi * 32 + __builtin_ctz(cur);
    cur &= cur - 1u;
    return j;
  };

  const float zs = a.scale * 1.4426950408889634f;

  // One chunk: selection, S^T, per-chunk softmax, PV.  Both row blocks run when either does.
  // The chunk that holds a block's own rows needs the causal mask; every other chunk takes a
  // branch-free path, so that one block's softmax can be scheduled between the other block's
  // MFMAs.
  auto compute = [&](int j, int stg, bool live) {
    bool sel[2];
    float wq[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      // The row's selection is ascending with a sentinel after entry k-1, so ptr stays <= k.
      const int e = rloc[b] * ks + ptr[b];
      sel[b] = live && sm.sidx[e] == (uint16_t)j;
      const float wv = static_cast<float>(sm.sw[e]);
      wq[b] = sel[b] ? wv : 0.f;
      ptr[b] += sel[b] ? 1 : 0;
    }
    if (!__any(sel[0] || sel[1])) return;
    const char* kbuf = sm.k[stg];
    const char* vbuf = sm.v[stg];
    // S^T of block b: lane (m, g) holds query row m and keys 16 kb + 4 g + rr.
    auto qk = [&](int b, float (&sv)[16]) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f32x4 acc = zero4();
        const T* krow = reinterpret_cast<const T*>(kbuf + (kb * 16 + m) * Lay::KLD) + g * (D / 4);
#pragma unroll
        for (int st = 0; st < NF; ++st) acc = Mfma<T>::mma(load_frag<T>(krow + st * KPL), qf[b][st], acc);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sv[kb * 4 + rr] = acc[rr];
      }
    };
    // Keys after the query in its own chunk are masked.
    auto mask = [&](int b, float (&sv)[16]) {
      const int ql = qpos[b] & 63;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (kb * 16 + 4 * g + rr > ql) sv[kb * 4 + rr] = -INFINITY;
    };
    // Per-chunk softmax of block b scaled by w_j / l_j, as the PV B operand.
    auto softmax = [&](int b, float (&sv)[16], typename Mfma<T>::frag (&pf)[NP]) {
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
      mx = col_max(mx) * zs;
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // v_exp_f32 directly: arguments are <= 0, results below 2^-126 may flush to zero.
        sv[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], zs, -mx));
        l += sv[i];
      }
      l = col_sum(l);                        // >= 1: the row maximum contributes exp2(0)
      const float f = wq[b] * __builtin_amdgcn_rcpf(l);
#pragma unroll
      for (int st = 0; st < NP; ++st) {
        if constexpr (KPL == 1) {
          pf[st] = sv[st] * f;
        } else {
#pragma unroll
          for (int z = 0; z < KPL; ++z) pf[st][z] = bf16_rne(sv[st * KPL + z] * f);
        }
      }
    };
    auto pv = [&](const typename Mfma<T>::frag (&p0)[NP], const typename Mfma<T>::frag (&p1)[NP]) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
#pragma unroll
        for (int st = 0; st < NP; ++st) {
          typename Mfma<T>::frag va;
          if constexpr (KPL == 1) va = v_frag_f32<Lay::VDB>(vbuf, m, g, db, st);
          else va = v_frag_bf16<Lay::VDB>(vbuf, m, g, db, st);
          acc_o[0][db] = Mfma<T>::mma(va, p0[st], acc_o[0][db]);
          acc_o[1][db] = Mfma<T>::mma(va, p1[st], acc_o[1][db]);
        }
      }
    };
    float s0[16], s1[16];
    typename Mfma<T>::frag pf0[NP], pf1[NP];
    if (j == crow[0] || j == crow[1]) {      // wave-uniform: rows of a block share a chunk
      qk(0, s0);
      qk(1, s1);
      if (j == crow[0]) mask(0, s0);
      if (j == crow[1]) mask(1, s1);
      softmax(0, s0, pf0);
      softmax(1, s1, pf1);
      pv(pf0, pf1);
    } else if constexpr (KPL == 1 || !kSplitPV) {
      qk(0, s0);
      qk(1, s1);
      softmax(0, s0, pf0);
      softmax(1, s1, pf1);
      pv(pf0, pf1);
    } else {
      // One basic block, ordered so that independent MFMA and VALU work can overlap: block 1's
      // S^T with block 0's softmax, block 0's PV with block 1's softmax (V fragments are read
      // once and kept for both blocks).
      qk(0, s0);
      qk(1, s1);
      softmax(0, s0, pf0);
      typename Mfma<T>::frag va[D / 16][NP];
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int st = 0; st < NP; ++st) va[db][st] = v_frag_bf16<Lay::VDB>(vbuf, m, g, db, st);
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int st = 0; st < NP; ++st) acc_o[0][db] = Mfma<T>::mma(va[db][st], pf0[st], acc_o[0][db]);
      softmax(1, s1, pf1);
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int st = 0; st < NP; ++st) acc_o[1][db] = Mfma<T>::mma(va[db][st], pf1[st], acc_o[1][db]);
    }
  };

  const int U = sm.nunion;
  int jl = -1;                               // last chunk returned by the iterator
  auto advance = [&]() -> int {
    const int j = next_chunk();
    if (j >= 0) jl = j;
    return j >= 0 ? j : jl;
  };
  if constexpr (STAGES == 1) {
    // One stage, nothing held in registers between chunks (fp32 at d = 128, where a chunk is
    // 64 KiB and two chunks in flight would not fit the registers): each chunk is copied into
    // the stage four vectors per tensor at a time, between two barriers, then computed.
    constexpr int NC = NV < 4 ? NV : 4;
    static_assert(NV % NC == 0, "copy pieces");
    for (int t = 0; t < U; ++t) {
      const int c = advance();
      const T* kc = kv_chunk<T, D>(Kb, static_cast<const T*>(a.key), bt, a.num_pages, a.H / a.G, kvh, c);
      const T* vc = kv_chunk<T, D>(Vb, static_cast<const T*>(a.val), bt, a.num_pages, a.H / a.G, kvh, c);
      __syncthreads();                       // the previous chunk's compute is done with the stage
#pragma unroll 1
      for (int u0 = 0; u0 < NV; u0 += NC) {
        u32x4 kr[NC], vr[NC];
#pragma unroll
        for (int u = 0; u < NC; ++u) {
          const int v = tid + NT * (u0 + u);
          kr[u] = *reinterpret_cast<const u32x4*>(kc + (size_t)v * VE);
          vr[u] = *reinterpret_cast<const u32x4*>(vc + (size_t)v * VE);
        }
#pragma unroll
        for (int u = 0; u < NC; ++u) {
          const int v = tid + NT * (u0 + u);
          const int row = v / Lay::VPR, p = v % Lay::VPR;
          *reinterpret_cast<u32x4*>(sm.k[0] + row * Lay::KLD + p * 16) = kr[u];
          const int e = p * VE;
          *reinterpret_cast<u32x4*>(sm.v[0] + (e >> 4) * Lay::VDB + row * (16 * (int)sizeof(T)) +
                                    (e & 15) * (int)sizeof(T)) = vr[u];
        }
      }
      __syncthreads();
      compute(c, 0, true);
    }
  } else if (U > 0) {
  // Loads and stores below are unconditional (past the end of the union they repeat its last
  // chunk) so that the compiler's wait counts stay exact across the loop.
  // Iteration t computes c_t from stage t%2 while c_{t+1} sits in register set (t+1)%2 and
  // c_{t+2} is loaded into set t%2; after the compute the registers of c_{t+1} go to stage
  // (t+1)%2 and one barrier publishes them.
    u32x4 kr[2][NV], vr[2][NV];
    const int c0 = advance();
    load_kv(c0, kr[0], vr[0]);
    store_kv(0, kr[0], vr[0]);
    int ca = c0, cb = advance();           // chunks t and t+1
    load_kv(cb, kr[1], vr[1]);
    __syncthreads();
    // Two chunks per trip (static register-set indexing); an odd U ends with an idle half.
    for (int t = 0; t < U; t += 2) {
      const int cc = advance();            // chunk t+2
      load_kv(cc, kr[0], vr[0]);
      compute(ca, 0, true);
      store_kv(1, kr[1], vr[1]);
      __syncthreads();
      const int cd = advance();            // chunk t+3
      load_kv(cd, kr[1], vr[1]);
      compute(cb, 1, t + 1 < U);
      store_kv(0, kr[0], vr[0]);
      __syncthreads();
      ca = cc;
      cb = cd;
    }
  }

  // O^T fragments: lane holds its rows' d = 16*db + 4g + rr.
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    T* op = static_cast<T*>(a.o) + (row0 + qpos[b]) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      typedef T vec4 __attribute__((ext_vector_type(4)));
      vec4 out;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) out[rr] = from_f32<T>(acc_o[b][db][rr]);
      *reinterpret_cast<vec4*>(op + db * 16 + 4 * g) = out;
    }
  }
}

// ------------------------------------------------------------------------------------------
// bf16, 32 < k <= 64: the k <= 32 kernel below with only the chunk indices staged in LDS (the
// weights, which a staged copy would double, are read from memory one match ahead: nw0 is the
// row's next match, nw1 the one after).  17 KiB of indices beside one K/V stage: two
// workgroups per CU.  (A copy of the selection kept entirely in memory, read per match, with
// two K/V stages was 12 % slower.)
template <int D, int QG, int KMAX>
struct BlockSelSmem64 {
  alignas(16) char k[64 * BlockKLayout<D>::LD];
  alignas(16) char v[AttnLayout<bf16, D>::VBYTES];
  int nunion;
  uint16_t sidx[QG * (KMAX + 1)];
};

// bf16, 32 < k <= 64: one 16-row MFMA block per wave, NW waves per 16*NW-query workgroup (eight
// by default: two workgroups, four waves per SIMD, share a CU).  Only the group's chunk indices
// are staged in LDS; each lane reads its row's weights from memory one match ahead.  One K/V
// stage, the next chunk held in registers, two barriers per chunk.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void chunk_attention_block64_kernel(const AttnArgs a) {
  constexpr int QG = 16 * NW, KMAX = 64;
  typedef BlockSelSmem64<D, QG, KMAX> Smem;
  typedef AttnLayout<bf16, D> Lay;
  constexpr int NF = D / 32;                 // QK^T steps over d
  constexpr int NP = 2;                      // PV steps over the 64 keys
  constexpr int VE = 8;                      // elements per 16-byte vector
  constexpr int NT = NW * 64;                // threads
  constexpr int NV = 64 * Lay::VPR / NT;     // 16-byte vectors per thread per tensor per chunk
  static_assert(NV >= 1 && (64 * Lay::VPR) % NT == 0, "chunk tile does not split over the threads");
  __shared__ Smem sm;
  extern __shared__ uint32_t bitmap[];       // ceil(N / 32) words

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int groups = a.L / QG;
  const uint32_t total = (uint32_t)a.B * a.H * groups;
  const uint32_t gid = xcd_remap(blockIdx.x, total);
  const int bh = gid / groups;
  const int q0 = (int)(gid % groups) * QG;   // first query position of the group
  const int c_last = (q0 + QG - 1) >> 6;     // last chunk a row of the group may select
  const int k = a.topk;
  const int ks = k + 1;                      // staged row stride (odd: rows hit distinct banks)
  const bf16* Kb = static_cast<const bf16*>(a.key) + (size_t)kv_pair(bh, a.H, a.G) * a.L * D;
  const bf16* Vb = static_cast<const bf16*>(a.val) + (size_t)kv_pair(bh, a.H, a.G) * a.L * D;
  const int32_t* bt = a.block_table ? a.block_table + (size_t)(bh / a.H) * a.bt_stride : nullptr;
  const int kvh = (bh % a.H) / a.G;
  const size_t row0 = (size_t)bh * a.L;

  // Stage the group's selections and build the union bitmap (causal chunks only).
  const int nwords = (c_last + 1 + 31) >> 5;
  for (int x = tid; x < nwords; x += NT) bitmap[x] = 0u;
  if (tid == 0) sm.nunion = 0;
  for (int r = tid; r < QG; r += NT) sm.sidx[r * ks + k] = (uint16_t)0xFFFF;   // end sentinel
  __syncthreads();
  for (int x = tid; x < QG * k; x += NT) {
    const int r = x / k, e = x - r * k;
    const int j = a.idx[(row0 + q0) * k + x];
    const bool ok = j >= 0 && j <= c_last;
    sm.sidx[r * ks + e] = ok ? (uint16_t)j : (uint16_t)0xFFFF;
    if (ok) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  {
    int cnt = 0;
    for (int x = tid; x < nwords; x += NT) cnt += __popc(bitmap[x]);
    cnt = (int)wave_sum((float)cnt);   // exact: at most 65536
    if (lane == 0) atomicAdd(&sm.nunion, cnt);
  }

  // This lane's row: 16 * wave + m of the group.
  const int rloc = 16 * wave + m, qpos = q0 + rloc, crow = qpos >> 6;
  int ptr = 0;
  const float* rw = a.w + (row0 + qpos) * k;
  float nw0 = rw[0], nw1 = k > 1 ? rw[1] : 0.f;
  bf16x8 qf[NF];
  {
    const bf16* qp = static_cast<const bf16*>(a.q) + (row0 + qpos) * D + g * (D / 4);
#pragma unroll
    for (int st = 0; st < NF; ++st) qf[st] = load_frag<bf16>(qp + st * 8);
  }
#pragma unroll
  for (int st = 0; st < NF; ++st) asm volatile("" ::"v"(qf[st]));
  f32x4 acc_o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc_o[db] = zero4();

  auto load_kv = [&](int j, u32x4 (&kr)[NV], u32x4 (&vr)[NV]) {
    const bf16* kc = kv_chunk<bf16, D>(Kb, static_cast<const bf16*>(a.key), bt, a.num_pages, a.H / a.G, kvh, j);
    const bf16* vc = kv_chunk<bf16, D>(Vb, static_cast<const bf16*>(a.val), bt, a.num_pages, a.H / a.G, kvh, j);
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
      *reinterpret_cast<u32x4*>(sm.k + BlockKLayout<D>::off(row, p)) = kr[u];
      const int e = p * VE;                  // first element of the vector
      *reinterpret_cast<u32x4*>(sm.v + (e >> 4) * Lay::VDB + row * 32 + (e & 15) * 2) = vr[u];
    }
  };

  __syncthreads();
  int wi = 0;
  uint32_t cur = bitmap[0];
  auto next_chunk = [&]() -> int {
    while (cur == 0u && wi + 1 < nwords) cur = bitmap[++wi];
    if (cur == 0u) return -1;
    const int j = wi * 32 + __builtin_ctz(cur);
    cur &= cur - 1u;
    return j;
  };

  const float zs = a.scale * 1.4426950408889634f;
  auto compute = [&](int j) {
    // The row's selection is ascending with a sentinel after entry k-1, so ptr stays <= k.
    const bool sel = sm.sidx[rloc * ks + ptr] == (uint16_t)j;
    const float wq = sel ? nw0 : 0.f;
    if (sel) {
      ++ptr;
      nw0 = nw1;
      nw1 = ptr + 1 < k ? rw[ptr + 1] : 0.f;
    }
    if (!__any(sel)) return;
    const char* kbuf = sm.k;
    const char* vbuf = sm.v;
    // Wave priority: the MFMA phases above the softmax, so that a SIMD's other waves fill the
    // MFMA gaps with their softmax rather than the reverse (about 1 % at 128K).
    __builtin_amdgcn_s_setprio(2);
    // S^T: lane (m, g) holds query row m and keys 16 kb + 4 g + rr.
    float sv[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = zero4();
#pragma unroll
      for (int st = 0; st < NF; ++st)
        acc = Mfma<bf16>::mma(load_frag<bf16>(reinterpret_cast<const bf16*>(kbuf + BlockKLayout<D>::off(kb * 16 + m, g * NF + st))), qf[st], acc);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sv[kb * 4 + rr] = acc[rr];
    }
    if (j == crow) {                         // wave-uniform: the block's rows share a chunk
      const int ql = qpos & 63;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (kb * 16 + 4 * g + rr > ql) sv[kb * 4 + rr] = -INFINITY;
    }
    __builtin_amdgcn_s_setprio(0);
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
    mx = col_max(mx) * zs;
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // v_exp_f32 directly: arguments are <= 0, results below 2^-126 may flush to zero.
      sv[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], zs, -mx));
      l += sv[i];
    }
    l = col_sum(l);                          // >= 1: the row maximum contributes exp2(0)
    const float f = wq * __builtin_amdgcn_rcpf(l);
    __builtin_amdgcn_s_setprio(2);
    bf16x8 pf[NP];
#pragma unroll
    for (int st = 0; st < NP; ++st)
#pragma unroll
      for (int z = 0; z < 8; ++z) pf[st][z] = bf16_rne(sv[st * 8 + z] * f);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int st = 0; st < NP; ++st)
        acc_o[db] = Mfma<bf16>::mma(v_frag_bf16<Lay::VDB>(vbuf, m, g, db, st), pf[st], acc_o[db]);
  };

  const int U = sm.nunion;
  int jl = -1;                               // last chunk returned by the iterator
  auto advance = [&]() -> int {
    const int j = next_chunk();
    if (j >= 0) jl = j;
    return j >= 0 ? j : jl;
  };
  // compute c_t; barrier; the registers holding c_{t+1} go to LDS and c_{t+2} is loaded into
  // them; barrier.  Loads and stores are unconditional (past the end of the union they repeat
  // its last chunk) so that the compiler's wait counts stay exact across the loop.
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

  // O^T fragments: lane holds its row's d = 16*db + 4g + rr.
  bf16* op = static_cast<bf16*>(a.o) + (row0 + qpos) * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    bf16x4 out;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) out[rr] = bf16_rne(acc_o[db][rr]);
    *reinterpret_cast<bf16x4*>(op + db * 16 + 4 * g) = out;
  }
}

// bf16, k <= 32: one 16-row MFMA block per wave, NW waves per 16*NW-query workgroup (eight by
// default).  A wave computes only the chunks its own 16 rows selected (no second block riding
// along), and a wave needs about half the registers of the two-block kernel above: at eight
// waves two workgroups (four waves per SIMD) share a CU.  Same staging and union walk as above:
// the group's selection staged in LDS, one LDS stage, the next chunk in registers, two barriers
// per chunk.  A row's result depends only on its own selection (rows that did not choose a
// chunk add exact zeros), so it is the same for every NW.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void chunk_attention_block_kernel(const AttnArgs a) {
  constexpr int QG = 16 * NW, KMAX = 32;
  typedef AttnSmem<bf16, D, QG, KMAX, 1> Smem;
  typedef AttnLayout<bf16, D> Lay;
  constexpr int NF = D / 32;                 // QK^T steps over d
  constexpr int NP = 2;                      // PV steps over the 64 keys
  constexpr int VE = 8;                      // elements per 16-byte vector
  constexpr int NT = NW * 64;                // threads
  constexpr int NV = 64 * Lay::VPR / NT;     // 16-byte vectors per thread per tensor per chunk
  static_assert(NV >= 1 && (64 * Lay::VPR) % NT == 0, "chunk tile does not split over the threads");
  __shared__ Smem sm;
  extern __shared__ uint32_t bitmap[];       // ceil(N / 32) words

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int groups = a.L / QG;
  const uint32_t total = (uint32_t)a.B * a.H * groups;
  const uint32_t gid = xcd_remap(blockIdx.x, total);
  const int bh = gid / groups;
  const int q0 = (int)(gid % groups) * QG;   // first query position of the group
  const int c_last = (q0 + QG - 1) >> 6;     // last chunk a row of the group may select
  const int k = a.topk;
  const int ks = k + 1;                      // staged row stride (odd: rows hit distinct banks)
  const bf16* Kb = static_cast<const bf16*>(a.key) + (size_t)kv_pair(bh, a.H, a.G) * a.L * D;
  const bf16* Vb = static_cast<const bf16*>(a.val) + (size_t)kv_pair(bh, a.H, a.G) * a.L * D;
  const int32_t* bt = a.block_table ? a.block_table + (size_t)(bh / a.H) * a.bt_stride : nullptr;
  const int kvh = (bh % a.H) / a.G;
  const size_t row0 = (size_t)bh * a.L;

  // Stage the group's selections and build the union bitmap (causal chunks only).
  const int nwords = (c_last + 1 + 31) >> 5;
  for (int x = tid; x < nwords; x += NT) bitmap[x] = 0u;
  if (tid == 0) sm.nunion = 0;
  for (int r = tid; r < QG; r += NT) sm.sidx[r * ks + k] = (uint16_t)0xFFFF;   // end sentinel
  __syncthreads();
  for (int x = tid; x < QG * k; x += NT) {
    const int r = x / k, e = x - r * k;
    const int j = a.idx[(row0 + q0) * k + x];
    const bool ok = j >= 0 && j <= c_last;
    sm.sidx[r * ks + e] = ok ? (uint16_t)j : (uint16_t)0xFFFF;
    sm.sw[r * ks + e] = a.w[(row0 + q0) * k + x];
    if (ok) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  {
    int cnt = 0;
    for (int x = tid; x < nwords; x += NT) cnt += __popc(bitmap[x]);
    cnt = (int)wave_sum((float)cnt);   // exact: at most 65536
    if (lane == 0) atomicAdd(&sm.nunion, cnt);
  }

  // This lane's row: 16 * wave + m of the group.
  const int rloc = 16 * wave + m, qpos = q0 + rloc, crow = qpos >> 6;
  int ptr = 0;
  bf16x8 qf[NF];
  {
    const bf16* qp = static_cast<const bf16*>(a.q) + (row0 + qpos) * D + g * (D / 4);
#pragma unroll
    for (int st = 0; st < NF; ++st) qf[st] = load_frag<bf16>(qp + st * 8);
  }
#pragma unroll
  for (int st = 0; st < NF; ++st) asm volatile("" ::"v"(qf[st]));
  f32x4 acc_o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc_o[db] = zero4();

  auto load_kv = [&](int j, u32x4 (&kr)[NV], u32x4 (&vr)[NV]) {
    const bf16* kc = kv_chunk<bf16, D>(Kb, static_cast<const bf16*>(a.key), bt, a.num_pages, a.H / a.G, kvh, j);
    const bf16* vc = kv_chunk<bf16, D>(Vb, static_cast<const bf16*>(a.val), bt, a.num_pages, a.H / a.G, kvh, j);
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
      *reinterpret_cast<u32x4*>(sm.k[0] + BlockKLayout<D>::off(row, p)) = kr[u];
      const int e = p * VE;                  // first element of the vector
      *reinterpret_cast<u32x4*>(sm.v[0] + (e >> 4) * Lay::VDB + row * 32 + (e & 15) * 2) = vr[u];
    }
  };

  __syncthreads();
  int wi = 0;
  uint32_t cur = bitmap[0];
  auto next_chunk = [&]() -> int {
    while (cur == 0u && wi + 1 < nwords) cur = bitmap[++wi];
    if (cur == 0u) return -1;
    const int j = wi * 32 + __builtin_ctz(cur);
    cur &= cur - 1u;
    return j;
  };

  const float zs = a.scale * 1.4426950408889634f;
  auto compute = [&](int j) {
    // The row's selection is ascending with a sentinel after entry k-1, so ptr stays <= k.
    const int e = rloc * ks + ptr;
    const bool sel = sm.sidx[e] == (uint16_t)j;
    const float wq = sel ? sm.sw[e] : 0.f;
    ptr += sel ? 1 : 0;
    if (!__any(sel)) return;
    const char* kbuf = sm.k[0];
    const char* vbuf = sm.v[0];
    // Wave priority: the MFMA phases above the softmax, so that a SIMD's other waves fill the
    // MFMA gaps with their softmax rather than the reverse (about 1 % at 128K).
    __builtin_amdgcn_s_setprio(2);
    // S^T: lane (m, g) holds query row m and keys 16 kb + 4 g + rr.
    float sv[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = zero4();
#pragma unroll
      for (int st = 0; st < NF; ++st)
        acc = Mfma<bf16>::mma(load_frag<bf16>(reinterpret_cast<const bf16*>(kbuf + BlockKLayout<D>::off(kb * 16 + m, g * NF + st))), qf[st], acc);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sv[kb * 4 + rr] = acc[rr];
    }
    if (j == crow) {                         // wave-uniform: the block's rows share a chunk
      const int ql = qpos & 63;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (kb * 16 + 4 * g + rr > ql) sv[kb * 4 + rr] = -INFINITY;
    }
    __builtin_amdgcn_s_setprio(0);
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
    mx = col_max(mx) * zs;
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // v_exp_f32 directly: arguments are <= 0, results below 2^-126 may flush to zero.
      sv[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], zs, -mx));
      l += sv[i];
    }
    l = col_sum(l);                          // >= 1: the row maximum contributes exp2(0)
    const float f = wq * __builtin_amdgcn_rcpf(l);
    __builtin_amdgcn_s_setprio(2);
    bf16x8 pf[NP];
#pragma unroll
    for (int st = 0; st < NP; ++st)
#pragma unroll
      for (int z = 0; z < 8; ++z) pf[st][z] = bf16_rne(sv[st * 8 + z] * f);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int st = 0; st < NP; ++st)
        acc_o[db] = Mfma<bf16>::mma(v_frag_bf16<Lay::VDB>(vbuf, m, g, db, st), pf[st], acc_o[db]);
  };

  const int U = sm.nunion;
  int jl = -1;                               // last chunk returned by the iterator
  auto advance = [&]() -> int {
    const int j = next_chunk();
    if (j >= 0) jl = j;
    return j >= 0 ? j : jl;
  };
  // compute c_t; barrier; the registers holding c_{t+1} go to LDS and c_{t+2} is loaded into
  // them; barrier.  Loads and stores are unconditional (past the end of the union they repeat
  // its last chunk) so that the compiler's wait counts stay exact across the loop.
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

  // O^T fragments: lane holds its row's d = 16*db + 4g + rr.
  bf16* op = static_cast<bf16*>(a.o) + (row0 + qpos) * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    bf16x4 out;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) out[rr] = bf16_rne(acc_o[db][rr]);
    *reinterpret_cast<bf16x4*>(op + db * 16 + 4 * g) = out;
  }
}

// ------------------------------------------------------------------------------------------
// Chunk-major mode (bf16), for selections whose rows share few chunks: the union walk above
// stages every chunk any row of a 128-row group chose and computes whole 16-row blocks, which on
// such inputs re-reads each chunk's K/V once per group and computes mostly discarded rows.  Here
// one (batch, head) pair at a time: the pair's selections are inverted into per-chunk lists
// (count, prefix, fill); each work item stages one chunk's K/V once and runs up to 128 of the
// rows that chose it, 16 per wave, writing w_j * o_j of that (row, slot) to a partial buffer;
// finally every row sums its partials in slot order.  The result of a (row, slot) does not
// depend on which rows share its tile, so the output is deterministic although the lists are
// filled in arrival order.

// Pair p of the batch (blockIdx.y of the kernels below): its tensors and its list buffers.
struct CmLists {
  const int32_t* idx;
  const float* w;
  uint32_t *cnt, *off, *cur, *toff, *ent, *desc;
};
__device__ __forceinline__ CmLists cm_lists(const CmArgs& a, int p) {
  const size_t bh = (size_t)a.pair0 + p, lk = (size_t)a.L * a.k;
  CmLists c;
  c.idx = a.idx + bh * lk;
  c.w = a.w + bh * lk;
  c.cnt = a.cnt + (size_t)p * a.N;
  c.off = a.off + (size_t)p * (a.N + 1);
  c.cur = a.cur + (size_t)p * a.N;
  c.toff = a.toff + (size_t)p * (a.N + 1);
  c.ent = a.ent + (size_t)p * lk * 2;
  c.desc = a.desc + (size_t)p * cm_max_items(lk, a.N) * 2;
  return c;
}
struct CmPair {
  const bf16 *q, *key, *val;
  const float* w;
  bf16* o;
  bf16* partial;
  const int32_t* bt;                           // the pair's block-table row (paged), else NULL
  int Hk, kvh;                                 // key/value heads per batch row, the pair's one
};
template <int D>
__device__ __forceinline__ CmPair cm_pair(const CmArgs& a, int p) {
  const size_t bh = (size_t)a.pair0 + p, b = bh / a.H, h = bh % a.H;
  const size_t ld = (size_t)a.L * D, lk = (size_t)a.L * a.k;
  CmPair c;
  c.Hk = a.H / a.G;
  c.kvh = (int)(h / a.G);
  const size_t kvbh = b * c.Hk + c.kvh;
  c.q = static_cast<const bf16*>(a.q) + bh * ld;
  if (a.bt) {                                  // pools: pages of every key/value head
    c.key = static_cast<const bf16*>(a.key);
    c.val = static_cast<const bf16*>(a.val);
    c.bt = a.bt + b * (size_t)a.bt_stride;
  } else {
    c.key = static_cast<const bf16*>(a.key) + kvbh * ld;
    c.val = static_cast<const bf16*>(a.val) + kvbh * ld;
    c.bt = nullptr;
  }
  c.w = a.w + bh * lk;
  c.o = static_cast<bf16*>(a.o) + bh * ld;
  c.partial = static_cast<bf16*>(a.partial) + (size_t)p * lk * D;
  return c;
}

__global__ __launch_bounds__(256) void cm_zero_kernel(uint32_t* cnt, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) cnt[i] = 0u;
}

// Selections per chunk.  Each workgroup takes a contiguous slice of the pair's (row, slot)
// entries and counts it into an LDS histogram first (nchunks <= kCmLdsChunks), so that a chunk
// costs one global atomic per workgroup instead of one per selection.
constexpr int kCmLdsChunks = 16384;
__global__ __launch_bounds__(256) void cm_count_kernel(const CmArgs a) {
  extern __shared__ uint32_t hist[];
  const CmLists c = cm_lists(a, blockIdx.y);
  const int32_t* idx = c.idx;
  uint32_t* cnt = c.cnt;
  const int n = a.L * a.k, nchunks = a.N;
  const int per = (n + gridDim.x - 1) / gridDim.x;
  const int b = min(n, (int)blockIdx.x * per), e = min(n, b + per);
  if (nchunks > kCmLdsChunks) {
    for (int i = b + threadIdx.x; i < e; i += 256) {
      const int j = idx[i];
      if (j >= 0 && j < nchunks) atomicAdd(&cnt[j], 1u);
    }
    return;
  }
  for (int j = threadIdx.x; j < nchunks; j += 256) hist[j] = 0u;
  __syncthreads();
  for (int i = b + threadIdx.x; i < e; i += 256) {
    const int j = idx[i];
    if (j >= 0 && j < nchunks) atomicAdd(&hist[j], 1u);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < nchunks; j += 256)
    if (hist[j]) atomicAdd(&cnt[j], hist[j]);
}

// One workgroup: off = exclusive prefix of cnt, cur = off, toff = exclusive prefix of
// ceil(cnt / kCmItem); off[N] and toff[N] are the totals.  Also the work items in order: item
// toff[j] + t of chunk j covers list entries off[j] + kCmItem t onward, at most kCmItem of them.
__global__ __launch_bounds__(1024) void cm_scan_kernel(const CmArgs a) {
  __shared__ uint32_t s_e[1024], s_t[1024];
  const CmLists c = cm_lists(a, blockIdx.x);
  const uint32_t* cnt = c.cnt;
  uint32_t *off = c.off, *cur = c.cur, *toff = c.toff, *desc = c.desc;
  const int N = a.N;
  const int t = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int b = min(N, t * per), e = min(N, b + per);
  uint32_t se = 0, st = 0;
  for (int i = b; i < e; ++i) {
    se += cnt[i];
    st += (cnt[i] + kCmItem - 1) / kCmItem;
  }
  s_e[t] = se;
  s_t[t] = st;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {         // inclusive Hillis-Steele scan
    const uint32_t ae = t >= d ? s_e[t - d] : 0u, at = t >= d ? s_t[t - d] : 0u;
    __syncthreads();
    s_e[t] += ae;
    s_t[t] += at;
    __syncthreads();
  }
  uint32_t pe = s_e[t] - se, pt = s_t[t] - st;
  for (int i = b; i < e; ++i) {
    off[i] = pe;
    cur[i] = pe;
    toff[i] = pt;
    const uint32_t ci = cnt[i], ni = (ci + kCmItem - 1) / kCmItem;
    for (uint32_t t2 = 0; t2 < ni; ++t2) {
      const uint32_t rows = min(ci - kCmItem * t2, (uint32_t)kCmItem);
      *reinterpret_cast<u32x2*>(desc + 2 * (size_t)(pt + t2)) = u32x2{pe + kCmItem * t2, ((uint32_t)i << 8) | rows};
    }
    pe += ci;
    pt += ni;
  }
  if (t == 1023) {
    off[N] = s_e[1023];
    toff[N] = s_t[1023];
  }
}

// List entries (row << 6 | slot, with the bits of the row's weight for that slot), grouped by chunk.  A workgroup reserves its share of each
// chunk's list with one global atomic (LDS histogram, then LDS cursors), over the same slices
// as cm_count_kernel.  The order inside a chunk's list is arrival order; results do not depend
// on it.
__global__ __launch_bounds__(256) void cm_fill_kernel(const CmArgs a) {
  extern __shared__ uint32_t sh[];             // hist[nchunks], base[nchunks]
  const CmLists c = cm_lists(a, blockIdx.y);
  const int32_t* idx = c.idx;
  const float* w = c.w;
  uint32_t *cur = c.cur, *ent = c.ent;
  const int n = a.L * a.k, k = a.k, nchunks = a.N;
  const int per = (n + gridDim.x - 1) / gridDim.x;
  const int b = min(n, (int)blockIdx.x * per), e = min(n, b + per);
  if (nchunks > kCmLdsChunks) {
    for (int i = b + threadIdx.x; i < e; i += 256) {
      const int j = idx[i];
      if (j >= 0 && j < nchunks) {
        const int r = i / k, s = i - r * k;
        *reinterpret_cast<u32x2*>(ent + 2 * (size_t)atomicAdd(&cur[j], 1u)) =
            u32x2{((uint32_t)r << 6) | (uint32_t)s, __float_as_uint(w[i])};
      }
    }
    return;
  }
  uint32_t* hist = sh;
  uint32_t* base = sh + nchunks;
  for (int j = threadIdx.x; j < nchunks; j += 256) hist[j] = 0u;
  __syncthreads();
  for (int i = b + threadIdx.x; i < e; i += 256) {
    const int j = idx[i];
    if (j >= 0 && j < nchunks) atomicAdd(&hist[j], 1u);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < nchunks; j += 256) {
    const uint32_t c = hist[j];
    if (c) base[j] = atomicAdd(&cur[j], c);
    hist[j] = 0u;                              // now this workgroup's cursor into its share
  }
  __syncthreads();
  for (int i = b + threadIdx.x; i < e; i += 256) {
    const int j = idx[i];
    if (j >= 0 && j < nchunks) {
      const int r = i / k, s = i - r * k;
      *reinterpret_cast<u32x2*>(ent + 2 * (size_t)(base[j] + atomicAdd(&hist[j], 1u))) =
          u32x2{((uint32_t)r << 6) | (uint32_t)s, __float_as_uint(w[i])};
    }
  }
}

// Persistent: workgroup b takes the contiguous run of work items [b I / G, (b + 1) I / G) of its
// pair (I items, G workgroups per pair); item i belongs to the chunk j with toff[j] <= i <
// toff[j + 1] and covers list entries off[j] + 128 (i - toff[j]) onward.  Consecutive items
// mostly belong to one chunk, whose K/V is then staged once for the whole run of them.
//
// C keys per chunk (64, or 32 / 128): S^T takes C / 16 key blocks, PV C / 32 steps; K rows keep
// the 64-key kernels' layout and V's d-blocks hold C rows.  For C != 64 the keys and values are
// either pages of C rows (whole chunks) or contiguous, where a partial last chunk is read with
// its rows clamped to the sequence: only rows of that chunk select it, as their own chunk, and the
// keys past each such row are masked.
template <int D, int C>
__global__ __launch_bounds__(512, C == 128 ? 2 : 4) void cm_attn_kernel(const CmArgs a) {
  constexpr int NT = 512;
  typedef AttnLayout<bf16, D> Lay;
  constexpr int NF = D / 32, NP = C / 32, NKB = C / 16, VE = 8;
  constexpr int NVT = C * Lay::VPR;            // 16-byte vectors per tensor per chunk
  constexpr int NV = (NVT + NT - 1) / NT;
  static_assert(NVT % NT == 0 || NT % NVT == 0, "chunk tile does not split over the threads");
  constexpr int VDB = C * 32 + 32;             // V d-block stride (C rows of 16 elements, padded)
  constexpr int kLogC = C == 32 ? 5 : C == 64 ? 6 : 7;
  static_assert(C == 32 || C == 64 || C == 128, "chunk of 32, 64 or 128 keys");
  // (64 keys: the padded-row tile size this kernel was tuned with; a smaller one changes its
  // register allocation and spills)
  __shared__ __attribute__((aligned(16))) char sk[C == 64 ? Lay::KBYTES : C * BlockKLayout<D>::LD];
  __shared__ __attribute__((aligned(16))) char sv_[(D / 16) * VDB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int N = a.N, k = a.k;
  const CmLists cl = cm_lists(a, blockIdx.y);
  const CmPair cp = cm_pair<D>(a, blockIdx.y);
  const uint32_t items = cl.toff[N];
  const bf16* Q = cp.q;
  const bf16* Kb = cp.key;
  const bf16* Vb = cp.val;
  bf16* P = cp.partial;
  const float zs = a.scale * 1.4426950408889634f;
  // Pipeline: while item n is computed, item n+1's K/V and q rows are in flight, its list entries
  // (row and weight) arrived one item earlier, and item n+2's descriptor one before that, so no
  // load waits on another issued in the same step (the vector memory counter completes in issue
  // order, so such a wait would also drain the prefetches).  Loads are unconditional, indices
  // clamped into the pair's items and the item's entries.
  uint32_t item = (uint32_t)((uint64_t)blockIdx.x * items / gridDim.x);
  const uint32_t end = (uint32_t)((uint64_t)(blockIdx.x + 1) * items / gridDim.x);
  if (item >= end) return;                     // workgroup-uniform
  auto ld_desc = [&](uint32_t it) -> u32x2 {
    return *reinterpret_cast<const u32x2*>(cl.desc + 2 * (size_t)min(it, end - 1u));
  };
  auto ld_ent = [&](const u32x2& dsc) -> u32x2 {   // this lane's entry of the item
    const uint32_t n = dsc[1] & 255u, t = (uint32_t)(16 * wave + m);
    return *reinterpret_cast<const u32x2*>(cl.ent + 2 * (size_t)(dsc[0] + min(t, n - 1u)));
  };
  u32x4 kr[NV], vr[NV];
  // Thread -> vector v of the chunk (row v / VPR); with fewer vectors than threads the spare
  // threads repeat the last one (same bytes to the same LDS address).
  auto vec_of = [&](int u) { return NVT >= NT ? tid + NT * u : min(tid, NVT - 1); };
  auto load_kv = [&](int j) {
    if constexpr (C == 64) {
      const bf16* kc = kv_chunk<bf16, D>(Kb, Kb, cp.bt, a.num_pages, cp.Hk, cp.kvh, j);
      const bf16* vc = kv_chunk<bf16, D>(Vb, Vb, cp.bt, a.num_pages, cp.Hk, cp.kvh, j);
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int v = vec_of(u);
        kr[u] = *reinterpret_cast<const u32x4*>(kc + (size_t)v * VE);
        vr[u] = *reinterpret_cast<const u32x4*>(vc + (size_t)v * VE);
      }
    } else if (cp.bt != nullptr) {             // pages of C rows (whole chunks only)
      const int pg = min(max(cp.bt[j], 0), a.num_pages - 1);
      const size_t base = ((size_t)pg * cp.Hk + cp.kvh) * C * D;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int v = vec_of(u);
        const size_t e = base + (size_t)v * VE;
        kr[u] = *reinterpret_cast<const u32x4*>(Kb + e);
        vr[u] = *reinterpret_cast<const u32x4*>(Vb + e);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int v = vec_of(u);
        const size_t row = (size_t)min(j * C + v / Lay::VPR, a.L - 1);
        const size_t e = row * D + (v % Lay::VPR) * VE;
        kr[u] = *reinterpret_cast<const u32x4*>(Kb + e);
        vr[u] = *reinterpret_cast<const u32x4*>(Vb + e);
      }
    }
  };
  auto load_q = [&](const u32x2& pw, bf16x8 (&qf_)[NF]) {
    const bf16* qp = Q + (size_t)(pw[0] >> 6) * D + g * (D / 4);
#pragma unroll
    for (int st = 0; st < NF; ++st) qf_[st] = load_frag<bf16>(qp + st * 8);
  };
  auto put_kv = [&]() {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = vec_of(u);
      const int row = v / Lay::VPR, p = v % Lay::VPR;
      *reinterpret_cast<u32x4*>(sk + BlockKLayout<D>::off(row, p)) = kr[u];
      const int e = p * VE;
      *reinterpret_cast<u32x4*>(sv_ + (e >> 4) * VDB + row * 32 + (e & 15) * 2) = vr[u];
    }
  };
  u32x2 dsc_c = ld_desc(item), dsc_n = ld_desc(item + 1), dsc_nn = ld_desc(item + 2), dsc_3;
  u32x2 pw_c = ld_ent(dsc_c), pw_n = ld_ent(dsc_n), pw_nn;
  bf16x8 qf[NF], qn[NF];
  load_q(pw_c, qf);
  load_kv((int)(dsc_c[1] >> 8));
  put_kv();
  __syncthreads();
  // Item n+1's K/V (when its chunk differs from item n's) and q rows, item n+2's entries, item
  // n+3's descriptor: the same loads in the same order before the loop and at the end of each
  // trip, so the waits in the loop are exact.
  auto prefetch = [&]() {
    if ((dsc_n[1] >> 8) != (dsc_c[1] >> 8)) load_kv((int)(dsc_n[1] >> 8));   // workgroup-uniform
    load_q(pw_n, qn);
    pw_nn = ld_ent(dsc_nn);
    dsc_3 = ld_desc(item + 3);
  };
  prefetch();
  for (;;) {
    const bool has_next = item + 1 < end;      // workgroup-uniform
    // Every lane computes: a lane past the item's last entry holds a copy of that entry and
    // writes the same partial, bit for bit, so the stores are unconditional and the memory
    // counter's waits stay exact.
    const int j = (int)(dsc_c[1] >> 8);
    {
      const int r = (int)(pw_c[0] >> 6), es = (int)(pw_c[0] & 63u);
      float sc[4 * NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int st = 0; st < NF; ++st)
          acc = Mfma<bf16>::mma(load_frag<bf16>(reinterpret_cast<const bf16*>(sk + BlockKLayout<D>::off(kb * 16 + m, g * NF + st))), qf[st], acc);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sc[kb * 4 + rr] = acc[rr];
      }
      if ((r >> kLogC) == j) {                 // the row's own chunk: keys after it are masked
        const int ql = r & (C - 1);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (kb * 16 + 4 * g + rr > ql) sc[kb * 4 + rr] = -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 4 * NKB; ++i) mx = fmaxf(mx, sc[i]);
      mx = col_max(mx) * zs;
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < 4 * NKB; ++i) {
        // v_exp_f32 directly: arguments are <= 0, results below 2^-126 may flush to zero.
        sc[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], zs, -mx));
        l += sc[i];
      }
      l = col_sum(l);                          // >= 1: the row maximum contributes exp2(0)
      const float f = __uint_as_float(pw_c[1]) * __builtin_amdgcn_rcpf(l);
      bf16x8 pf[NP];
#pragma unroll
      for (int st = 0; st < NP; ++st)
#pragma unroll
        for (int z = 0; z < 8; ++z) pf[st][z] = bf16_rne(sc[st * 8 + z] * f);
      f32x4 acc_o[D / 16];
#pragma unroll
      for (int db = 0; db < D / 16; ++db) acc_o[db] = zero4();
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int st = 0; st < NP; ++st)
          acc_o[db] = Mfma<bf16>::mma(v_frag_bf16<VDB>(sv_, m, g, db, st), pf[st], acc_o[db]);
      bf16* op = P + ((size_t)r * k + es) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        bf16x4 out;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) out[rr] = bf16_rne(acc_o[db][rr]);
        *reinterpret_cast<bf16x4*>(op + db * 16 + 4 * g) = out;
      }
    }
    // Keep the hand-over of the prefetched registers below the compute: a copy scheduled into
    // it would wait there for the prefetches.
    __builtin_amdgcn_sched_barrier(0);
    if (!has_next) break;
    ++item;
    const bool new_chunk = (dsc_n[1] >> 8) != (dsc_c[1] >> 8);   // workgroup-uniform
#pragma unroll
    for (int st = 0; st < NF; ++st) qf[st] = qn[st];
    pw_c = pw_n;
    pw_n = pw_nn;
    dsc_c = dsc_n;
    dsc_n = dsc_nn;
    dsc_nn = dsc_3;
    if (new_chunk) {
      __syncthreads();                         // the previous chunk's LDS reads are done
      put_kv();
      __syncthreads();
    }
    prefetch();
  }
}

// o[r] = sum over the row's slots, in slot order, of its partials (fp32), rounded once.  The
// selection holds min(k, c + 1) chunks at the front of row r's list (c = r / C, the row's
// chunk), so those are the valid slots.  Eight elements per thread, D / 8 threads per row.
template <int D>
__global__ __launch_bounds__(256) void cm_reduce_kernel(const CmArgs a) {
  constexpr int TPR = D / 8;                   // threads per row
  const int r = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  if (r >= a.L) return;
  const CmPair cp = cm_pair<D>(a, blockIdx.y);
  const int nv = min(a.k, r / a.C + 1);
  const bf16* P = cp.partial + (size_t)r * a.k * D + t * 8;
  float acc[8] = {};
  int e = 0;
  for (; e + 8 <= nv; e += 8) {                // eight independent loads in flight
    bf16x8 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(P + (size_t)(e + u) * D));
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int z = 0; z < 8; ++z) acc[z] += to_f32(x[u][z]);
  }
  for (; e < nv; ++e) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(P + (size_t)e * D);
#pragma unroll
    for (int z = 0; z < 8; ++z) acc[z] += to_f32(x[z]);
  }
  bf16x8 out;
#pragma unroll
  for (int z = 0; z < 8; ++z) out[z] = bf16_rne(acc[z]);
  *reinterpret_cast<bf16x8*>(cp.o + (size_t)r * D + t * 8) = out;
}

template <int D>
hipError_t launch_chunk_attention_cm(const CmArgs& a, hipStream_t st) {
  const int n = a.L * a.k, np = a.npairs;
  const int gb = min((n + 8191) / 8192, 1024);   // workgroups per pair over the entries, 8192+ each
  const bool lds = a.N <= kCmLdsChunks;
  const int nz = a.N * np;
  hipLaunchKernelGGL(cm_zero_kernel, dim3(min((nz + 255) / 256, 1024)), dim3(256), 0, st, a.cnt, nz);
  hipLaunchKernelGGL(cm_count_kernel, dim3(gb, np), dim3(256), lds ? (size_t)a.N * 4 : 0, st, a);
  hipLaunchKernelGGL(cm_scan_kernel, dim3(np), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(cm_fill_kernel, dim3(gb, np), dim3(256), lds ? (size_t)a.N * 8 : 0, st, a);
  // 512 persistent workgroups in all (at least 64 per pair), each pair's own taking its items.
  const int wpp = max(64, 512 / np);
  if (a.C == 32) hipLaunchKernelGGL((cm_attn_kernel<D, 32>), dim3(wpp, np), dim3(512), 0, st, a);
  else if (a.C == 128) hipLaunchKernelGGL((cm_attn_kernel<D, 128>), dim3(wpp, np), dim3(512), 0, st, a);
  else hipLaunchKernelGGL((cm_attn_kernel<D, 64>), dim3(wpp, np), dim3(512), 0, st, a);
  constexpr int RPB = 256 / (D / 8);           // rows per reduce workgroup
  hipLaunchKernelGGL((cm_reduce_kernel<D>), dim3((a.L + RPB - 1) / RPB, np), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Union probe for the automatic mode: workgroup s takes sampled 128-row group s * total / S and
// adds the number of distinct chunks its rows selected to *out (zeroed by the caller's launch).
__global__ __launch_bounds__(256) void union_probe_kernel(const int32_t* idx, int H, int L, int k, int gpr,
                                                          uint32_t total_groups, uint32_t* out) {
  extern __shared__ uint32_t bits[];
  const uint32_t gsel = (uint32_t)(((uint64_t)blockIdx.x * total_groups) / gridDim.x);
  const int bh = (int)(gsel / gpr), q0 = (int)(gsel % gpr) * 128;
  const int rows = min(128, L - q0);
  const int nwords = ((q0 + rows - 1) / 64 + 1 + 31) / 32;
  for (int x = threadIdx.x; x < nwords; x += 256) bits[x] = 0u;
  __syncthreads();
  const int32_t* p = idx + ((size_t)bh * L + q0) * k;
  for (int x = threadIdx.x; x < rows * k; x += 256) {
    const int j = p[x];
    if (j >= 0 && j < nwords * 32) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  uint32_t c = 0;
  for (int x = threadIdx.x; x < nwords; x += 256) c += __popc(bits[x]);
  if (c) atomicAdd(out, c);
  (void)H;
}

hipError_t launch_union_probe(const int32_t* idx, int B, int H, int L, int k, uint32_t* total, int* groups,
                              hipStream_t st) {
  const int gpr = (L + 127) / 128;             // 128-row groups per (batch, head)
  const uint32_t all = (uint32_t)B * H * gpr;
  const int S = all < 256u ? (int)all : 256;
  *groups = S;
  const size_t bm = (size_t)(((L + 63) / 64 + 31) / 32) * 4;
  hipLaunchKernelGGL(cm_zero_kernel, dim3(1), dim3(256), 0, st, total, 1);
  hipLaunchKernelGGL(union_probe_kernel, dim3(S), dim3(256), bm, st, idx, H, L, k, gpr, all, total);
  return hipGetLastError();
}

template hipError_t launch_chunk_attention_cm<64>(const CmArgs&, hipStream_t);
template hipError_t launch_chunk_attention_cm<128>(const CmArgs&, hipStream_t);

// Queries per workgroup: bf16 takes a.q_tile (16, 32, 64 or 128 one-block waves of 16 rows; the
// caller guarantees L % q_tile == 0); at 128, two workgroups share a CU, with the selection staged
// in LDS for k <= 32 and its chunk indices only for k <= 64.  fp32 (a correctness path) keeps
// the two-block kernel: 256 queries (8 waves, k <= 32), 128 (4 waves) or 64 with two stages, so
// that the staged selection fits LDS.  Every choice gives the same result.
template <int D, int NW>
static void launch_block(const AttnArgs& a, uint32_t bhs, size_t bm, hipStream_t st) {
  const dim3 grid(bhs * (a.L / (16 * NW))), block(64 * NW);
  if (a.topk <= 32)
    hipLaunchKernelGGL((chunk_attention_block_kernel<D, NW>), grid, block, bm, st, a);
  else
    hipLaunchKernelGGL((chunk_attention_block64_kernel<D, NW>), grid, block, bm, st, a);
}

template <typename T, int D>
hipError_t launch_chunk_attention(const AttnArgs& a, hipStream_t st) {
  const uint32_t bhs = (uint32_t)a.B * a.H;
  const size_t bm = (size_t)((a.N + 31) / 32) * 4;   // union bitmap (dynamic LDS)
  if constexpr (sizeof(T) == 2) {
    switch (a.q_tile) {
      case 16: launch_block<D, 1>(a, bhs, bm, st); break;
      case 32: launch_block<D, 2>(a, bhs, bm, st); break;
      case 64: launch_block<D, 4>(a, bhs, bm, st); break;
      default: launch_block<D, 8>(a, bhs, bm, st); break;
    }
  } else if constexpr (D == 128) {              // 32 KiB per tensor per chunk: 64-query groups, one stage
    hipLaunchKernelGGL((chunk_attention_kernel<T, D, 2, 64, 1>), dim3(bhs * (a.L / 64)), dim3(128), bm, st, a);
  } else {
    if (a.topk <= 32 && a.L % 256 == 0) {
      hipLaunchKernelGGL((chunk_attention_kernel<T, D, 8, 32, 2>), dim3(bhs * (a.L / 256)), dim3(512), bm, st, a);
    } else if (a.L % 128 == 0) {
      hipLaunchKernelGGL((chunk_attention_kernel<T, D, 4, 64, 2>), dim3(bhs * (a.L / 128)), dim3(256), bm, st, a);
    } else {
      hipLaunchKernelGGL((chunk_attention_kernel<T, D, 2, 64, 2>), dim3(bhs * (a.L / 64)), dim3(128), bm, st, a);
    }
  }
  return hipGetLastError();
}

template hipError_t launch_chunk_attention<bf16, 64>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<bf16, 128>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<float, 64>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<float, 128>(const AttnArgs&, hipStream_t);

}  // namespace hils
