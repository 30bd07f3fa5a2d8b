// Chunk selection for prefill, bf16 with k <= 64: one wave per 64-query tile, eight tiles per
// workgroup for k <= 32, four for 32 < k <= 64.
//
// Method: [HiLS-Attention model page, "Model Description"] every query scores all causal chunks
// through their landmark keys, keeps the k best and weights them with a softmax over those
// scores; [HiLS Attention explainer (molayo1419.me), "Engineering details", Q-Cal item] scoring
// uses q~ = q + W_up W_down h.  Ties keep the smaller chunk index; the output is in ascending
// chunk order with -1 / 0 padding when fewer than k chunks exist.
//
// With C = 64 the 64 queries of tile c share the candidate set {0..c}, so scoring is a GEMM
// [64 queries x d] x [d x (c+1)] done with v_mfma_f32_32x32x16_bf16: A = 32 landmark rows,
// B = q~ of 32 queries (registers, two column blocks).  The d order of the contraction is the
// one in which the Q-Cal MFMA delivers its output, so q~ is formed in registers.  The tiles of
// a workgroup are consecutive chunks of one (batch, head), so they need the same landmark
// blocks: each block is loaded once (global -> registers several blocks ahead -> LDS) and read
// by all the workgroup's waves.  The output of block jb holds, at lane (col, half), query
// column col and landmark rows 8(e/4) + 4 half + e%4; one v_permlane32_swap per element pair
// moves both halves of a query's 32 rows into one lane, so lane l owns query 32*(l/32) + l%32
// and all of its scores.
//
// Exact top-k in two passes over the landmarks:
//   pass 1: per slot the two largest scores, a slot being a landmark row within a 32-row block
//           (k <= 32: 32 slots) or a row and the block's parity (k <= 64: 64 slots); the kq-th
//           largest of these 2 x slots values is reached by at least kq distinct chunks, so it
//           bounds the kq-th largest score from below (tau).  They are kept in the MFMA output layout
//           and swapped into the query's lane once, at the end.  Skipped when all candidates
//           fit the list.
//   pass 2: every score >= tau is appended, in ascending chunk order, to the query's LDS list
//           ([position][query] so the 64 lanes write distinct banks).  A list that could
//           overflow is cut to its exact top-kq first and tau is raised above the cut value
//           (later chunks lose ties); with the tight tau of pass 1 this is rare.
//   final:  the kq-th largest theta of the list (a sorting network for lists of up to 64
//           entries, else a bisection over the order-preserving 32-bit keys); entries > theta
//           and the first (kq - #>theta) entries == theta are kept in list order, then the
//           inter-chunk softmax.  The wave's output rows are staged in LDS and leave as 16-byte
//           stores.
// Scores are finite by contract: this file is compiled with -fno-honor-nans, so max/min skip
// NaN quieting.
#include <float.h>

#include <type_traits>

#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Per k range: tiles per workgroup, list capacity per query (>= kq + 8) and the number of
// pass-1 slots per query (rows of a 32-landmark block, times the block parity for k > 32).
// Both take one workgroup per CU (LDS); k <= 64 has one wave per SIMD, with room for 512
// registers.
template <int KQ> struct SelCfg;
template <> struct SelCfg<32> { static constexpr int kTiles = 8, kCap = 47, kPar = 1; };
template <> struct SelCfg<64> { static constexpr int kTiles = 4, kCap = 88, kPar = 2; };

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void cx_desc(float& a, float& b) {
  const float hi = fmaxf(a, b), lo = fminf(a, b);
  a = hi;
  b = lo;
}

// Bitonic sort of N values, descending (static network, registers only).
template <int N>
__device__ __forceinline__ void sort_desc(float (&x)[N]) {
#pragma unroll
  for (int kk = 2; kk <= N; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ jj;
        if (l > i) {
          if ((i & kk) == 0) cx_desc(x[i], x[l]);
          else cx_desc(x[l], x[i]);
        }
      }
    }
  }
}

// Sort a bitonic sequence of N values into descending order.
template <int N>
__device__ __forceinline__ void bitonic_merge_desc(float (&x)[N]) {
#pragma unroll
  for (int jj = N >> 1; jj > 0; jj >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & jj) == 0) cx_desc(x[i], x[i + jj]);
  }
}

// x[kk - 1] of a descending array for a runtime kk in [1, N]: the minimum of its first kk
// entries (a select-by-index chain would be lowered to a scratch-memory array).
template <int N>
__device__ __forceinline__ float pick(const float (&x)[N], int kk) {
  float r = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) r = fminf(r, i < kk ? x[i] : INFINITY);
  return r;
}

// Wave w takes 64-query tile t_top - w, so the tiles of a workgroup are consecutive tiles of one
// (batch, head) and need the same landmark blocks.  Chunks of C = 32 or 128 keys: a tile's rows
// have the candidates 0 .. (row / C), the same for the whole tile at C = 128 (two tiles per
// chunk) and one more for its second half at C = 32; the tile is scored against the candidates
// of its last row and each query masks the landmarks past its own chunk.

typedef __attribute__((address_space(3))) void lds_void;

// Landmark rows in the ring are stored with their 16-byte vectors permuted (vector v of row r at
// position v ^ ring_swz(r)), so that the 16 rows of one MFMA operand read fall on distinct banks.
template <int D>
__device__ __forceinline__ int ring_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

template <int D, int KQ>
struct GroupSmem {
  static constexpr int kCap = SelCfg<KQ>::kCap;
  static constexpr int RB = 2 * D;             // landmark row bytes
  alignas(16) char ring[2][32 * RB];           // 32-landmark blocks, even / odd block index
  struct {
    float s[kCap * 64];                        // [row][query] candidate scores
    uint16_t j[kCap * 64];                     // [row][query] candidate chunks
  } w[SelCfg<KQ>::kTiles];
};

}  // namespace

// QV = 1: the Q-Cal rank is a multiple of 8 and at most 32 (the one Q-Cal form compiled, which
// keeps the prologue's registers to that form); QV = 0: any rank, chosen at run time.
template <int D, int KQ, int QV>
__global__ __launch_bounds__(64 * SelCfg<KQ>::kTiles) void select_fast_kernel(const SelectArgs a) {
  constexpr int kTiles = SelCfg<KQ>::kTiles, kCap = SelCfg<KQ>::kCap, kPar = SelCfg<KQ>::kPar;
  constexpr int NS = D / 16;                   // MFMA k-steps over d
  typedef GroupSmem<D, KQ> Smem;
  static_assert(sizeof(Smem) <= 160 * 1024, "LDS");
  __shared__ Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int lc = 31 - __builtin_clz((unsigned)a.C);   // log2 of the chunk size
  const int T = a.L >> 6;                      // 64-query tiles per (batch, head)
  const int G = (T + kTiles - 1) / kTiles;     // tile groups per (batch, head)
  const uint32_t total = (uint32_t)a.B * a.H * G;
  const uint32_t grp = xcd_remap(blockIdx.x, total);
  const int bh = grp / G;
  const int t_top = T - 1 - kTiles * (int)(grp % G);     // longest groups first
  // A wave past tile 0 (T not a multiple of kTiles) runs tile 0 again and writes nothing.
  const bool active = t_top - wave >= 0;
  const int q0 = max(t_top - wave, 0) * 64;
  const int c_top = (64 * t_top + 63) >> lc;   // the group's last candidate chunk
  const int b = bh / a.H, hd = bh % a.H;
  const int n_cand = ((q0 + 63) >> lc) + 1;    // candidates of the tile's last row
  // Candidates of query col and col + 32 (MFMA output columns), and of query `lane` (after the
  // lane swap each lane owns one query); equal to n_cand at C >= 64.
  const int nc0 = ((q0 + col) >> lc) + 1, nc1 = ((q0 + 32 + col) >> lc) + 1;
  const int nql = ((q0 + lane) >> lc) + 1;
  const int nb = (n_cand + 31) >> 5;           // this tile's 32-landmark blocks
  const int nbg = (c_top + 1 + 31) >> 5;       // blocks the group sweeps
  const int kq = min(a.k, nql);
  const bf16* Q = static_cast<const bf16*>(a.q) + (size_t)bh * a.L * D;
  const bf16* LM = static_cast<const bf16*>(a.lmk) + (size_t)kv_pair(bh, a.H, a.G) * a.N * D;
  // This lane's list: row i at ls[64 i], lj[64 i].
  float* ls = &sm.w[wave].s[lane];
  uint16_t* lj = &sm.w[wave].j[lane];

  // ---------------- q~ as the B operand ------------------------------------------------------
  // Lane (col, half) holds query 32 cb + col.  The d order of the scoring contraction is the
  // order in which the Q-Cal MFMA below delivers its output rows: k-slot z of step s at lane
  // half h is d(s, h, z) = 16 s + 8 (z / 4) + 4 h + z % 4, so q~ is formed in registers.  The
  // landmark rows are laid out in LDS in the same order (see the ring).
  bf16x8 qf[2][NS];
  auto load_q = [&](int cb) {
    const bf16* qrow = Q + (size_t)(q0 + 32 * cb + col) * D;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(qrow + 16 * st + 4 * half);
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(qrow + 16 * st + 8 + 4 * half);
      qf[cb][st] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  // delta_q^T[d][query] = sum_r W_up[hd*D + d][r] t[query][r]; t (fp32) is split into three bf16
  // parts so that every product is exact and the sum is accumulated in fp32.  VEC: r is a
  // multiple of 8, so every 8-slot run is a whole 16-byte piece of a row.  Loads are
  // unconditional (indices clamped into the row, values past r zeroed after the load) and each
  // variant is straight-line code, so the compiler keeps the loads in flight together.
  auto qcal = [&](auto vec_c, auto nrs_c) {
    constexpr bool VEC = decltype(vec_c)::value;
    constexpr int NRS = decltype(nrs_c)::value;   // 16-wide r steps: r <= 16 NRS
    const int r = a.r, nrs = (r + 15) >> 4;
    const bf16* WU = static_cast<const bf16*>(a.w_up) + (size_t)hd * D * r;
    // W_up fragment of rows 32 db + col, r-slots 16 rs + 8 half + z.
    auto wfrag = [&](int db, int rs) {
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
    // One query block at a time (registers): t split in three, then the D / 32 row blocks of
    // W_up, the next one's fragments loading while the current one's MFMAs run.
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      load_q(cb);
      bf16x8 tb[3][NRS];
      const float* tq = a.tcode + ((size_t)b * a.L + q0 + 32 * cb + col) * r;
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
      bf16x8 wcur[NRS], wnext[NRS];
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) wcur[rs] = wfrag(0, rs);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        if (db + 1 < D / 32) {
#pragma unroll
          for (int rs = 0; rs < NRS; ++rs) wnext[rs] = wfrag(db + 1, rs);
        }
        f32x16 acc = {};
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) {
          if (rs < nrs) {
#pragma unroll
            for (int p = 0; p < 3; ++p) acc = mfma32(wcur[rs], tb[p][rs], acc);
          }
        }
        // acc[e]: query 32 cb + col, d = 32 db + 8 (e / 4) + 4 half + e % 4 = d(2 db + e / 8,
        // half, e % 8).
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          bf16x8& f = qf[cb][2 * db + e / 8];
          f[e % 8] = bf16_rne(to_f32(f[e % 8]) + acc[e]);
        }
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) wcur[rs] = wnext[rs];
      }
    }
  };
  if constexpr (QV == 1) {
    qcal(std::true_type{}, std::integral_constant<int, 2>{});
  } else if (a.r > 0) {
    constexpr std::integral_constant<int, 2> r32{};
    constexpr std::integral_constant<int, 4> r64{};
    if ((a.r & 7) == 0) {
      if (a.r <= 32) qcal(std::true_type{}, r32);
      else qcal(std::true_type{}, r64);
    } else {
      if (a.r <= 32) qcal(std::false_type{}, r32);
      else qcal(std::false_type{}, r64);
    }
  } else {
    load_q(0);
    load_q(1);
  }

  // ---------------- landmark ring ------------------------------------------------------------
  // Block jb = landmark rows 32 jb .. 32 jb + 31 (clamped to the group's last candidate).  Each
  // block goes global -> registers -> LDS: every wave loads D / kTiles bytes per lane of it into
  // register stage jb % kDepth, and writes them to ring slot jb & 1 one step before the block is
  // used, so kDepth blocks are in flight while the group computes.  Loads and stores are
  // unconditional (clamped rows) so the compiler counts the loads in flight instead of draining
  // them.  In LDS, row r's 16-byte vector v = 2 s + h holds d(s, h, 0..7), stored at position
  // v ^ ring_swz(r): a global 8-byte piece d = 16 s + 8 g + 4 h' + (0..3) goes to vector
  // 2 s + h', bytes 8 g .. 8 g + 7.
  constexpr int kDepth = 4;
  constexpr int LB = D / kTiles;               // bytes per lane per block: 8, 16 or 32
  constexpr int UB = LB >= 16 ? 16 : 8;        // bytes per load
  constexpr int NPW = LB / UB;                 // loads per lane per block
  typedef typename std::conditional<UB == 16, u32x4, u32x2>::type unit_t;
  static_assert(32 * Smem::RB == 64 * kTiles * LB, "block size");
  unit_t stage[kDepth][NPW];
  auto unit_off = [&](int u) { return (u * kTiles + wave) * 64 * UB + UB * lane; };  // row-major
  auto gload = [&](int jb, unit_t (&dst)[NPW]) {
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
      const int o = unit_off(u);
      const int row = min(32 * jb + o / Smem::RB, c_top);
      dst[u] = *reinterpret_cast<const unit_t*>(LM + (size_t)row * D + (o % Smem::RB) / 2);
    }
  };
  auto lput = [&](int slot, const unit_t (&src)[NPW]) {
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
      const int o = unit_off(u), r = o / Smem::RB, e0 = (o % Smem::RB) / 2;   // first d
#pragma unroll
      for (int hp = 0; hp < UB / 8; ++hp) {    // 8-byte pieces d = e0 + 4 hp .. + 3
        const int d0 = e0 + 4 * hp, st = d0 / 16, g = (d0 / 8) & 1, h = (d0 / 4) & 1;
        char* dst = sm.ring[slot] + r * Smem::RB + 16 * ((2 * st + h) ^ ring_swz<D>(r)) + 8 * g;
        *reinterpret_cast<u32x2*>(dst) = u32x2{src[u][2 * hp], src[u][2 * hp + 1]};
      }
    }
  };
  // The group walks its blocks in order; f(jb, block) runs once the block is in LDS.  The walk
  // is rounded up to whole kDepth steps; every wave takes every barrier; f skips blocks past
  // its own tile.
  auto sweep = [&](auto&& f) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) gload(u, stage[u]);
    __syncthreads();                           // no wave still reads the ring
    lput(0, stage[0]);
    gload(kDepth, stage[0]);
    for (int jb0 = 0; jb0 < nbg; jb0 += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int jb = jb0 + u;
        __syncthreads();                       // block jb is in LDS; slot (jb + 1) & 1 is free
        lput((jb + 1) & 1, stage[(u + 1) % kDepth]);
        gload(jb + 1 + kDepth, stage[(u + 1) % kDepth]);
        if (jb < nbg) f(jb, sm.ring[jb & 1]);
      }
    }
  };

  // ---------------- scoring of one 32-landmark block ---------------------------------------
  // A operand: lane (col, half) takes row col, d(s, half, 0..7).  Rows past the last
  // candidate hold later landmarks or repeat the group's last one; their scores are masked.
  auto read_a = [&](const char* blk, bf16x8 (&af)[NS]) {
    const char* rp = blk + col * Smem::RB;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      af[s] = *reinterpret_cast<const bf16x8*>(rp + 16 * ((2 * s + half) ^ ring_swz<D>(col)));
  };
  // The scoring MFMAs run at a raised wave priority and the VALU work on their results at the
  // normal one, so that a SIMD's other wave fills the MFMA gaps (3 % at 512K with k = 64).
  auto mma_block = [&](const bf16x8 (&af)[NS], f32x16& acc0, f32x16& acc1) {
    __builtin_amdgcn_s_setprio(2);
    acc0 = f32x16{};
    acc1 = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      acc0 = mfma32(af[s], qf[0][s], acc0);
      acc1 = mfma32(af[s], qf[1][s], acc1);
    }
  };
  // The block's scores for this lane's query, handed to f(row, score) in ascending row order
  // (rows past the last candidate read -inf).  acc0/acc1 hold column blocks 0/1 with rows
  // 8(e/4) + 4 half + e%4; after the swap lanes 0-31 hold both row halves of column block 0
  // and lanes 32-63 both row halves of column block 1.
  auto for_scores = [&](auto last_block, int jb, const f32x16& acc0, const f32x16& acc1, auto&& f) {
    constexpr bool last = decltype(last_block)::value;
    const int lim = nql - 32 * jb;
#pragma unroll
    for (int grp4 = 0; grp4 < 4; ++grp4) {
      float x[4], y[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = 4 * grp4 + t;
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0[e]), __float_as_uint(acc1[e]),
                                                        false, false);
        x[t] = __uint_as_float(r[0]);          // row 8 grp4 + t
        y[t] = __uint_as_float(r[1]);          // row 8 grp4 + 4 + t
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) f(8 * grp4 + t, (last && 8 * grp4 + t >= lim) ? -INFINITY : x[t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) f(8 * grp4 + 4 + t, (last && 8 * grp4 + 4 + t >= lim) ? -INFINITY : y[t]);
    }
  };

  // ---------------- pass 1: lower bound tau of the kq-th largest score ---------------------
  // Slots: the 32 rows of a block (k <= 32), or rows times block parity (k <= 64).  The two
  // largest scores per slot are kept in the MFMA output layout: m[p][e] for query col (rows
  // 8(e/4) + 4 half + e%4), m[p][16 + e] for query col + 32; the lanes' halves are swapped once
  // at the end, giving each lane 64 kPar values of its query.
  float tau = -FLT_MAX;                        // every finite score passes; masked ones do not
  if (c_top + 1 > kCap) {                      // group-uniform: some tile has more than kCap
    const bool mine = n_cand > kCap;
    float m1[kPar][32], m2[kPar][32];
#pragma unroll
    for (int p = 0; p < kPar; ++p)
#pragma unroll
      for (int i = 0; i < 32; ++i) m1[p][i] = m2[p][i] = -INFINITY;
    auto slots = [&](auto par, int jb, const f32x16& acc0, const f32x16& acc1) {
      constexpr int P = decltype(par)::value;
      auto top2 = [&](int i, float v) {
        m2[P][i] = __builtin_amdgcn_fmed3f(m1[P][i], m2[P][i], v);
        m1[P][i] = fmaxf(m1[P][i], v);
      };
      if (jb == nb - 1) {
        const int lim0 = nc0 - 32 * jb, lim1 = nc1 - 32 * jb;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 8 * (e / 4) + 4 * half + e % 4;
          top2(e, row >= lim0 ? -INFINITY : acc0[e]);
          top2(16 + e, row >= lim1 ? -INFINITY : acc1[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          top2(e, acc0[e]);
          top2(16 + e, acc1[e]);
        }
      }
    };
    sweep([&](int jb, const char* blk) {
      if (!mine || jb >= nb) return;
      bf16x8 af[NS];
      read_a(blk, af);
      f32x16 acc0, acc1;
      mma_block(af, acc0, acc1);
      __builtin_amdgcn_s_setprio(0);
      if (kPar == 2 && (jb & 1)) slots(std::integral_constant<int, kPar - 1>{}, jb, acc0, acc1);
      else slots(std::integral_constant<int, 0>{}, jb, acc0, acc1);
    });
    if (mine) {
#pragma unroll
      for (int p = 0; p < kPar; ++p)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m1[p][e]),
                                                           __float_as_uint(m1[p][16 + e]), false, false);
          m1[p][e] = __uint_as_float(r1[0]);
          m1[p][16 + e] = __uint_as_float(r1[1]);
          const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m2[p][e]),
                                                           __float_as_uint(m2[p][16 + e]), false, false);
          m2[p][e] = __uint_as_float(r2[0]);
          m2[p][16 + e] = __uint_as_float(r2[1]);
        }
      // Top 32 kPar of the 64 kPar values: sort the first and second maxima, merge, pick kq-th.
      constexpr int NM = 32 * kPar;
      float u1[NM], u2[NM];
#pragma unroll
      for (int p = 0; p < kPar; ++p)
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          u1[32 * p + i] = m1[p][i];
          u2[32 * p + i] = m2[p][i];
        }
      sort_desc<NM>(u1);
      sort_desc<NM>(u2);
#pragma unroll
      for (int i = 0; i < NM; ++i) u1[i] = fmaxf(u1[i], u2[NM - 1 - i]);
      bitonic_merge_desc<NM>(u1);
      tau = pick<NM>(u1, kq);
    }
  }

  // ---------------- pass 2: collect the candidates ------------------------------------------
  // Every score >= tau is appended, in chunk order, to the lane's list in LDS.
  int cnt = 0;
  {
    // Make room for the next 8 scores: a list that would overflow is cut to its exact top kq
    // first (rare: lists end near kq + a few).  theta = kq-th largest key, bit by bit from the
    // top, counting list entries in LDS; entries > theta and the first kq - #(> theta)
    // entries == theta stay, in list order.  The cut runs in rolled loops over the list in LDS
    // so that it stays small in the unrolled sweep.
    auto make_room = [&](const float (&sc)[32], int h0) {
      if (__any(cnt + 8 > kCap)) {
        int np = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) np += sc[h0 + i] >= tau ? 1 : 0;
        if (cnt + np > kCap) {
          uint32_t th = 0u;
#pragma unroll 1
          for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = th | (1u << bit);
            int n = 0;
#pragma unroll 1
            for (int i = 0; i < cnt; ++i) n += f32_key(ls[64 * i]) >= cand ? 1 : 0;
            if (n >= kq) th = cand;
          }
          int ngt = 0;
#pragma unroll 1
          for (int i = 0; i < cnt; ++i) ngt += f32_key(ls[64 * i]) > th ? 1 : 0;
          const int m_eq = kq - ngt;
          int w = 0, eq = 0;
#pragma unroll 1
          for (int i = 0; i < cnt; ++i) {
            const float v = ls[64 * i];
            const uint32_t key = f32_key(v);
            bool keep = key > th;
            if (key == th) {
              keep = eq < m_eq;
              ++eq;
            }
            if (keep) {                        // w <= i: entries move towards the front
              const uint16_t jv = lj[64 * i];
              ls[64 * w] = v;
              lj[64 * w] = jv;
              ++w;
            }
          }
          cnt = w;
          tau = key_f32(th + 1u);              // later chunks must beat theta strictly
        }
      }
    };
    float sc[32];
    auto keep = [&](int i, float v) { sc[i] = v; };
    auto collect = [&](int jb, const f32x16& acc0, const f32x16& acc1) {
      if (jb == nb - 1) for_scores(std::true_type{}, jb, acc0, acc1, keep);
      else for_scores(std::false_type{}, jb, acc0, acc1, keep);
#pragma unroll
      for (int h0 = 0; h0 < 32; h0 += 8) {     // at most 8 appends after each check
        // Most groups of 8 hold no candidate for any of the wave's queries: one wave-wide test
        // of the group maximum skips the eight per-score branches.
        float gm = sc[h0];
#pragma unroll
        for (int i = 1; i < 8; ++i) gm = fmaxf(gm, sc[h0 + i]);
        if (!__any(gm >= tau)) continue;
        make_room(sc, h0);
#pragma unroll
        for (int i = h0; i < h0 + 8; ++i) {
          if (sc[i] >= tau) {
            ls[64 * cnt] = sc[i];
            lj[64 * cnt] = (uint16_t)(32 * jb + i);
            ++cnt;
          }
        }
      }
    };
    sweep([&](int jb, const char* blk) {
      if (jb >= nb) return;
      bf16x8 af[NS];
      read_a(blk, af);
      f32x16 acc0, acc1;
      mma_block(af, acc0, acc1);
      __builtin_amdgcn_s_setprio(0);
      collect(jb, acc0, acc1);
    });
  }

  // ---------------- final top-kq and inter-chunk softmax ------------------------------------
  // The list (cnt <= kCap entries, chunk order) is read into registers once.
  float ev[kCap];
  int ej[kCap];
#pragma unroll
  for (int i = 0; i < kCap; ++i) {
    ev[i] = i < cnt ? ls[64 * i] : -INFINITY;
    ej[i] = i < cnt ? (int)lj[64 * i] : 0;
  }
  float theta, top;
  if constexpr (kCap <= 64) {
    float v[64];                               // kCap entries padded to the sort width
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = i < kCap ? ev[i] : -INFINITY;
    sort_desc<64>(v);
    top = v[0];
    theta = pick<64>(v, kq);
  } else {
    // theta = kq-th largest key, bit by bit over the list in registers (padding is -inf).
    top = ev[0];
#pragma unroll
    for (int i = 1; i < kCap; ++i) top = fmaxf(top, ev[i]);
    uint32_t th = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = th | (1u << bit);
      int n = 0;
#pragma unroll
      for (int i = 0; i < kCap; ++i) n += f32_key(ev[i]) >= cand ? 1 : 0;
      if (n >= kq) th = cand;
    }
    theta = key_f32(th);
  }
  // Entries > theta, then the first kq - #(> theta) entries == theta in chunk order.
  int ngt = 0;
#pragma unroll
  for (int i = 0; i < kCap; ++i) ngt += ev[i] > theta ? 1 : 0;   // padding is -inf
  const int m_eq = kq - ngt;
  bool kept[kCap];
  {
    int eq = 0;
#pragma unroll
    for (int i = 0; i < kCap; ++i) {
      bool keep = ev[i] > theta;
      if (i < cnt && ev[i] == theta) {
        keep = eq < m_eq;
        ++eq;
      }
      kept[i] = keep;
    }
  }
  if (!active) return;
  const float zs = a.scale * 1.4426950408889634f;   // scale * log2(e)
  float esum = 0.f;
#pragma unroll
  for (int i = 0; i < kCap; ++i) {
    ev[i] = kept[i] ? exp2f((ev[i] - top) * zs) : 0.f;
    esum += ev[i];
  }
  const float inv = 1.f / esum;
  // The output rows go through LDS: the lane's kept entries (chunk order) to positions 0..kq-1
  // of its staging row (stride k + 1 words; position k takes the writes of entries not kept),
  // padding (-1, 0) to kq..k-1.  The wave's 64 rows are contiguous in idx and w, so they then
  // leave as 16-byte stores.  The staging rows reuse the wave's list space, already read.
  static_assert(sizeof(sm.w[0]) >= 2 * 64 * (KQ + 1) * sizeof(float), "staging rows");
  const int S = a.k + 1;
  int* st_i = reinterpret_cast<int*>(&sm.w[wave]);
  float* st_w = reinterpret_cast<float*>(st_i + 64 * S);
  {
    int* ri = st_i + lane * S;
    float* rw = st_w + lane * S;
    int pos = 0;
#pragma unroll
    for (int i = 0; i < kCap; ++i) {
      ri[pos] = ej[i];
      rw[pos] = ev[i] * inv;
      pos += kept[i] ? 1 : 0;
    }
    for (int p = kq; p < a.k; ++p) {
      ri[p] = -1;
      rw[p] = 0.f;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's rows are in LDS
  const int nw = 64 * a.k;                     // words of the wave's rows (a multiple of 4)
  const uint32_t mk = ((1u << 20) + a.k - 1) / a.k;   // word / k == (word * mk) >> 20, word < 4096
  const size_t obase = ((size_t)bh * a.L + q0) * a.k;
  for (int w0 = 4 * lane; w0 < nw; w0 += 256) {
    u32x4 vi;
    f32x4 vw;
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      const int word = w0 + z;
      const int row = (int)(((uint32_t)word * mk) >> 20);
      const int at = row * S + (word - row * a.k);
      vi[z] = (uint32_t)st_i[at];
      vw[z] = st_w[at];
    }
    *reinterpret_cast<u32x4*>(a.idx + obase + w0) = vi;
    *reinterpret_cast<f32x4*>(a.w + obase + w0) = vw;
  }
}

template <int D, int KQ>
void launch_select_fast_k(const SelectArgs& a, hipStream_t st) {
  constexpr int T = SelCfg<KQ>::kTiles;
  const uint32_t groups = (uint32_t)a.B * a.H * ((a.L / 64 + T - 1) / T);
  if (a.r > 0 && a.r % 8 == 0 && a.r <= 32)
    hipLaunchKernelGGL((select_fast_kernel<D, KQ, 1>), dim3(groups), dim3(64 * T), 0, st, a);
  else
    hipLaunchKernelGGL((select_fast_kernel<D, KQ, 0>), dim3(groups), dim3(64 * T), 0, st, a);
}

template <int D>
hipError_t launch_select_fast(const SelectArgs& a, hipStream_t st) {
  if (a.k <= 32) launch_select_fast_k<D, 32>(a, st);
  else launch_select_fast_k<D, 64>(a, st);
  return hipGetLastError();
}

template hipError_t launch_select_fast<64>(const SelectArgs&, hipStream_t);
template hipError_t launch_select_fast<128>(const SelectArgs&, hipStream_t);

}  // namespace hils
