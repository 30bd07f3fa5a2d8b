// Intra-chunk attention and fusion for prefill.
//
// Method: [HiLS Attention explainer (molayo1419.me), "Core idea", level 2] ordinary softmax
// attention over the tokens of each selected chunk; ["HiLS Attention Extrapolates 64x at 90%
// Retrieval Accuracy"] each chunk is attended independently and the per-chunk outputs are summed
// with the inter-chunk weights.  Because every chunk's softmax is normalised on its own, the
// fused output is sum_j (w_j / l_j) * sum_t exp(a_t - m_j) v_t: no rescaling across chunks.
//
// Kernel (the pages' "load the union once" idea, designed afresh for wave64/MFMA): a workgroup
// takes 32*NW consecutive queries of one (batch, head) - several 64-query chunks - and walks the
// union of their selected chunks in ascending order.  Each union chunk's K and V (row-major,
// padded so MFMA operand reads hit distinct LDS banks) are staged once in LDS and shared by all
// waves; V fragments are read with gfx950's LDS transpose read.  Wave w owns rows 32w..32w+31 as
// two 16-row blocks and skips any block none of whose rows selected the chunk.
//   S^T[key][q] = K . Q^T  : A = K rows (LDS), B = raw q (registers);
//                            lane (m, g) holds query m and keys 16*kb + 4g + rr;
//   O^T[d][q] += V^T . P'^T: A = V^T via transpose reads, B = P' = p * (w_j / l_j) (registers).
// Each row's selection (ascending, from the selection kernel) is consumed through a pointer
// kept in registers; the next entry is fetched from global memory while other chunks run.
#include <float.h>
#include <limits.h>

#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

// One stage holds a chunk's K and V.  Direct global->LDS loads write whole 1 KiB runs, so any
// layout is chosen by where each lane loads from:
//   K: row-major, 16-byte vectors XOR-swizzled inside each row (slot (row, p) holds logical
//      vector p ^ swz_k(row)) so the MFMA operand reads of 16 rows hit distinct banks;
//   V: d-block-major, [d/16][row][16 elements], so a transpose read of 8 rows x 32 bytes covers
//      all banks once and every d-block sits at a fixed offset from the first.
template <typename T, int D>
struct AttnLayout {
  static constexpr int RB = D * (int)sizeof(T);                 // row bytes
  static constexpr int VPR = RB / 16;                          // 16-byte vectors per row
  static constexpr int RPL = RB >= 256 ? 1 : 256 / RB;         // rows per 256-byte bank line
  static constexpr int TILE = 64 * RB;                         // bytes of K (or V) per chunk
  // chunks in flight (one computed, the others loading): 3 when they fit in LDS, else 2
  static constexpr int STAGES = 3 * 2 * TILE + 8192 <= 160 * 1024 ? 3 : 2;
  static constexpr int SPR = (int)sizeof(T);                   // V: 16-byte slots per row per d-block
  static constexpr int VDB = 64 * 16 * (int)sizeof(T);         // V: bytes per d-block
  __device__ static int swz_k(int row) { return (row / RPL) % (VPR < 16 ? VPR : 16); }
};

// Selection of the group's rows, staged once: chunk index (u16, 0xFFFF = padding) and weight.
template <typename T, int D, int QG, int KMAX>
struct AttnSmem {
  static constexpr int BITMAP_WORDS = (sizeof(T) == 4 && D == 128) ? 512 : 2048;
  char kv[AttnLayout<T, D>::STAGES][2][AttnLayout<T, D>::TILE];
  uint32_t bitmap[BITMAP_WORDS];
  uint16_t sidx[QG * (KMAX + 1)];
  float sw[QG * (KMAX + 1)];
};

typedef __attribute__((address_space(3))) void lds_void;

template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag k_frag(const char* kbuf, int row, int g, int st) {
  typedef AttnLayout<T, D> Lay;
  constexpr int KPL = Mfma<T>::KPL, VE = 16 / (int)sizeof(T);
  const int e = g * (D / 4) + st * KPL;          // first element of the fragment
  const int phys = (e / VE) ^ Lay::swz_k(row);
  const char* p = kbuf + row * Lay::RB + phys * 16 + (e % VE) * (int)sizeof(T);
  return load_frag<T>(reinterpret_cast<const T*>(p));
}

// PV A-operand fragments (bf16) for one step st, all 8 d-blocks of D = 128: slot z of lane group
// g holds key 16*(i/4) + 4g + i%4 with i = 8*st + z (the S^T output layout).  Transpose read: lane
// L of each 16-lane group supplies 4 elements of row (base + L/4), columns 4*(L%4).. of a d-block,
// and lane i of the group receives column i of those four rows.  The reads are issued from one
// asm block that also waits for them: the compiler cannot tell that these LDS reads do not
// overlap in-flight global->LDS loads and would otherwise wait for all of those first.
// addr: LDS byte address of row (32*st + 4g + L/4), column 4*(L%4) of d-block 0; d-block db is at
// +2048*db and rows +16 at +512.
__device__ __forceinline__ void v_frags_d128(uint32_t addr, bf16x8 (&fr)[8]) {
  u32x2 o[16];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:512\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %3, %16 offset:2560\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %5, %16 offset:4608\n\t"
      "ds_read_b64_tr_b16 %6, %16 offset:6144\n\t"
      "ds_read_b64_tr_b16 %7, %16 offset:6656\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:8192\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:8704\n\t"
      "ds_read_b64_tr_b16 %10, %16 offset:10240\n\t"
      "ds_read_b64_tr_b16 %11, %16 offset:10752\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:12288\n\t"
      "ds_read_b64_tr_b16 %13, %16 offset:12800\n\t"
      "ds_read_b64_tr_b16 %14, %16 offset:14336\n\t"
      "ds_read_b64_tr_b16 %15, %16 offset:14848\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
        "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]),
        "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
      : "v"(addr)
      : "memory");
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const bf16x4 lo = __builtin_bit_cast(bf16x4, o[2 * db]), hi = __builtin_bit_cast(bf16x4, o[2 * db + 1]);
    fr[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}
// Same for D = 64 (4 d-blocks).
__device__ __forceinline__ void v_frags_d64(uint32_t addr, bf16x8 (&fr)[4]) {
  u32x2 o[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:512\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:2560\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:4096\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:4608\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:6144\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:6656\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
        "=&v"(o[7])
      : "v"(addr)
      : "memory");
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const bf16x4 lo = __builtin_bit_cast(bf16x4, o[2 * db]), hi = __builtin_bit_cast(bf16x4, o[2 * db + 1]);
    fr[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}
// K fragments (bf16) of one 16-key block for all N steps over d, read in one asm block that
// also waits for them (same reason as above).  addr[st]: LDS byte address of the lane's 16 bytes.
__device__ __forceinline__ void k_frags4(const uint32_t (&addr)[4], bf16x8 (&fr)[4]) {
  u32x4 o[4];
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) fr[i] = __builtin_bit_cast(bf16x8, o[i]);
}
__device__ __forceinline__ void k_frags2(const uint32_t (&addr)[2], bf16x8 (&fr)[2]) {
  u32x4 o[2];
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1])
      : "v"(addr[0]), "v"(addr[1])
      : "memory");
#pragma unroll
  for (int i = 0; i < 2; ++i) fr[i] = __builtin_bit_cast(bf16x8, o[i]);
}

// fp32: one element per step, key 16*(st/4) + 4g + st%4, column 16*db + lane16.
template <int D>
__device__ __forceinline__ float v_frag_f32(const char* vbuf, int lane16, int g, int db, int st) {
  const int row = 16 * (st >> 2) + 4 * g + (st & 3);
  return *reinterpret_cast<const float*>(vbuf + db * (64 * 64) + row * 64 + lane16 * 4);
}

template <typename T, int D, int NW, int KMAX>
__global__ __launch_bounds__(NW * 64, 1) void chunk_attention_kernel(const AttnArgs a) {
  constexpr int QG = 32 * NW;                // queries per workgroup
  typedef AttnSmem<T, D, QG, KMAX> Smem;
  typedef AttnLayout<T, D> Lay;
  constexpr int KPL = Mfma<T>::KPL;
  constexpr int NF = D / 4 / KPL;            // QK^T steps over d
  constexpr int NP = 64 / Mfma<T>::K;        // PV steps over the 64 keys
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int NT = NW * 64;                // threads
  constexpr int IPW = Lay::VPR / NW;         // direct-load instructions per wave per tensor
  constexpr int NLD = 2 * IPW;               // direct loads per thread per chunk
  constexpr int STAGES = Lay::STAGES;
  static_assert(Lay::VPR % NW == 0, "chunk tile does not split over the waves");
  __shared__ Smem sm;

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
  const T* Kb = static_cast<const T*>(a.key) + (size_t)bh * a.L * D;
  const T* Vb = static_cast<const T*>(a.val) + (size_t)bh * a.L * D;
  const size_t row0 = (size_t)bh * a.L;

  // Stage the group's selections and build the union bitmap (causal chunks only).
  const int nwords = (c_last + 1 + 31) >> 5;
  for (int x = tid; x < nwords; x += NT) sm.bitmap[x] = 0u;
  __syncthreads();
  for (int x = tid; x < QG * k; x += NT) {
    const int r = x / k, e = x - r * k;
    const int j = a.idx[(row0 + q0) * k + x];
    const bool ok = j >= 0 && j <= c_last;
    sm.sidx[r * ks + e] = ok ? (uint16_t)j : (uint16_t)0xFFFF;
    sm.sw[r * ks + e] = a.w[(row0 + q0) * k + x];
    if (ok) atomicOr(&sm.bitmap[j >> 5], 1u << (j & 31));
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
  // Use the query fragments once here so their loads retire before the pipelined loop starts
  // (otherwise every iteration would wait for all outstanding loads before the first MFMA).
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int st = 0; st < NF; ++st) asm volatile("" ::"v"(qf[b][st]));
  f32x4 acc_o[2][D / 16];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc_o[b][db] = zero4();

  // Direct global->LDS loads of chunk j into stage stg: wave w writes 1 KiB runs w*IPW.. of each
  // tensor; the source address of each lane places its 16 bytes in the layout described above.
  auto issue_kv = [&](int j, int stg) {
    const T* kc = Kb + (size_t)j * 64 * D;
    const T* vc = Vb + (size_t)j * 64 * D;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int run = wave * IPW + i;
      const int s = run * 64 + lane;
      const int row = s / Lay::VPR, p = s % Lay::VPR;
      __builtin_amdgcn_global_load_lds((const void*)(kc + row * D + (p ^ Lay::swz_k(row)) * VE),
                                       (lds_void*)(sm.kv[stg][0] + run * 1024), 16, 0, 0);
      const int vdb = s / (64 * Lay::SPR), vw = s % (64 * Lay::SPR);
      const int vrow = vw / Lay::SPR, vpart = vw % Lay::SPR;
      __builtin_amdgcn_global_load_lds((const void*)(vc + vrow * D + 16 * vdb + vpart * VE),
                                       (lds_void*)(sm.kv[stg][1] + run * 1024), 16, 0, 0);
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

  // Pipeline: chunk t is computed while the next STAGES-1 chunks load.  Every iteration issues
  // NLD loads for one chunk (past the end of the union, a repeat of the current one), and loads
  // retire in issue order, so after chunk t's loads come exactly (STAGES-2)*NLD others when
  // chunk t is needed.
  const float zs = a.scale * 1.4426950408889634f;
  int j = next_chunk();
  int jn = (STAGES == 3 && j >= 0) ? next_chunk() : -1;
  if (j >= 0) {
    issue_kv(j, 0);
    if constexpr (STAGES == 3) issue_kv(jn >= 0 ? jn : j, 1);
  }
  int stg = 0;
  while (j >= 0) {
    int j2;
    if constexpr (STAGES == 3) {
      j2 = jn >= 0 ? next_chunk() : -1;
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");
    } else {
      j2 = next_chunk();
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // Workgroup barrier without a memory fence (a fence would also wait for the loads still in
    // flight): this wave's LDS reads of the previous stage are done and its loads of chunk j have
    // landed, so after the barrier chunk j is complete and the previous stage is free.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // the next chunk goes to the stage computed in the previous iteration (all waves are past it)
    issue_kv(j2 >= 0 ? j2 : j, stg == 0 ? STAGES - 1 : stg - 1);

    bool sel[2];
    float wq[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int e = rloc[b] * ks + ptr[b];
      sel[b] = ptr[b] < k && sm.sidx[e] == (uint16_t)j;
      wq[b] = sel[b] ? sm.sw[e] : 0.f;
      ptr[b] += sel[b] ? 1 : 0;
    }
    const char* kbuf = sm.kv[stg][0];
    const char* vbuf = sm.kv[stg][1];
    const bool act[2] = {__any(sel[0]) != 0, __any(sel[1]) != 0};
    if (act[0] || act[1]) {
      // S^T for the active row blocks; each K fragment is read once and used by both blocks.
      float s[2][16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int row = kb * 16 + m;
        typename Mfma<T>::frag kf[NF];
        if constexpr (KPL == 1) {
#pragma unroll
          for (int st = 0; st < NF; ++st) kf[st] = k_frag<T, D>(kbuf, row, g, st);
        } else {
          uint32_t ad[NF];
          const uint32_t base = (uint32_t)(size_t)(lds_void*)kbuf + row * Lay::RB;
#pragma unroll
          for (int st = 0; st < NF; ++st) ad[st] = base + ((((g * (D / 4) + st * KPL) / VE) ^ Lay::swz_k(row)) << 4);
          if constexpr (NF == 4) k_frags4(ad, kf);
          else k_frags2(ad, kf);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (!act[b]) continue;
          f32x4 acc = zero4();
#pragma unroll
          for (int st = 0; st < NF; ++st) acc = Mfma<T>::mma(kf[st], qf[b][st], acc);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) s[b][kb * 4 + rr] = acc[rr];
        }
      }
      // Per-chunk softmax of each active block; P' = p * (w / l) is the PV B operand.
      typename Mfma<T>::frag pf[2][NP];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (!act[b]) continue;
        if (j == crow[b]) {     // own chunk: keys after the query are masked
          const int ql = qpos[b] & 63;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (kb * 16 + 4 * g + rr > ql) s[b][kb * 4 + rr] = -INFINITY;
        }
        float mx = s[b][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
        mx = col_max(mx);
        float l = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[b][i] = exp2f((s[b][i] - mx) * zs);
          l += s[b][i];
        }
        l = col_sum(l);
        const float f = wq[b] / l;
#pragma unroll
        for (int st = 0; st < NP; ++st) {
          if constexpr (KPL == 1) {
            pf[b][st] = s[b][st] * f;
          } else {
#pragma unroll
            for (int z = 0; z < KPL; ++z) pf[b][st][z] = bf16_rne(s[b][st * KPL + z] * f);
          }
        }
      }
      // O^T += V^T P'^T; each V fragment is read once and used by both blocks.
      if constexpr (KPL == 1) {
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
          for (int st = 0; st < NP; ++st) {
            const float va = v_frag_f32<D>(vbuf, m, g, db, st);
#pragma unroll
            for (int b = 0; b < 2; ++b)
              if (act[b]) acc_o[b][db] = Mfma<T>::mma(va, pf[b][st], acc_o[b][db]);
          }
      } else {
        const uint32_t vaddr = (uint32_t)(size_t)(lds_void*)vbuf + (4 * g + (m >> 2)) * 32 + 8 * (m & 3);
#pragma unroll
        for (int st = 0; st < NP; ++st) {
          bf16x8 fr[D / 16];
          if constexpr (D == 128) v_frags_d128(vaddr + 1024 * st, fr);
          else v_frags_d64(vaddr + 1024 * st, fr);
#pragma unroll
          for (int db = 0; db < D / 16; ++db)
#pragma unroll
            for (int b = 0; b < 2; ++b)
              if (act[b]) acc_o[b][db] = Mfma<T>::mma(fr[db], pf[b][st], acc_o[b][db]);
        }
      }
    }
    stg = stg == STAGES - 1 ? 0 : stg + 1;
    if constexpr (STAGES == 3) {
      j = jn;
      jn = j2;
    } else {
      j = j2;
    }
  }
  // all of this workgroup's global->LDS loads have retired before it exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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

// Queries per workgroup: 256 (8 waves) when k <= 32, else 128 (4 waves), so that the staged
// selection fits LDS next to three chunk stages; 64 when the sequence does not split that way.
template <typename T, int D>
hipError_t launch_chunk_attention(const AttnArgs& a, hipStream_t st) {
  const uint32_t bhs = (uint32_t)a.B * a.H;
  if constexpr (sizeof(T) == 4 && D == 128) {   // 32 KiB per tensor per chunk: 64-query groups
    hipLaunchKernelGGL((chunk_attention_kernel<T, D, 2, 64>), dim3(bhs * (a.L / 64)), dim3(128), 0, st, a);
  } else {
    if (a.topk <= 32 && a.L % 256 == 0) {
      hipLaunchKernelGGL((chunk_attention_kernel<T, D, 8, 32>), dim3(bhs * (a.L / 256)), dim3(512), 0, st, a);
    } else if (a.L % 128 == 0) {
      hipLaunchKernelGGL((chunk_attention_kernel<T, D, 4, 64>), dim3(bhs * (a.L / 128)), dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL((chunk_attention_kernel<T, D, 2, 64>), dim3(bhs * (a.L / 64)), dim3(128), 0, st, a);
    }
  }
  return hipGetLastError();
}

template hipError_t launch_chunk_attention<bf16, 64>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<bf16, 128>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<float, 64>(const AttnArgs&, hipStream_t);
template hipError_t launch_chunk_attention<float, 128>(const AttnArgs&, hipStream_t);

}  // namespace hils
