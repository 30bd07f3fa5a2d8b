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
// B = q~ of 32 queries (registers, two column blocks).  The tiles of a workgroup are
// consecutive chunks of one (batch, head), so they need the same landmark blocks: each block is
// loaded once, straight from global memory into an LDS ring (global_load_lds_dwordx4, no
// registers), and read by all the workgroup's waves.  The output of block jb holds, at lane (col, half),
// query column col and landmark rows 8(e/4) + 4 half + e%4; one v_permlane32_swap per element
// pair moves both halves of a query's 32 rows into one lane, so lane l owns query
// 32*(l/32) + l%32 and all of its scores.
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
//           overflow is cut to its exact top-kq first (from a register copy of its keys) and
//           tau is raised above the cut value (later chunks lose ties); with the tight tau of
//           pass 1 this is rare.
//   final:  the kq-th largest theta of the list (a sorting network for lists of up to 64
//           entries, else a bisection over the order-preserving 32-bit keys); entries > theta
//           and the first (kq - #>theta) entries == theta are kept in list order, then the
//           inter-chunk softmax.
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
// k <= 64 takes one workgroup per CU (LDS), so one wave per SIMD, with room for 512 registers.
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

// Wave w takes the 64-query tile of chunk c_top - w, so the tiles of a workgroup are consecutive
// chunks of one (batch, head) and need the same landmark blocks.

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
  static constexpr int QLD = D + 8;            // q~ staging row stride (elements)
  alignas(16) char ring[2][32 * RB];           // 32-landmark blocks, even / odd block index
  union {
    bf16 qt[64 * QLD];                         // q~ [query][d], before the sweeps
    struct {
      float s[kCap * 64];                      // [position][query] candidate scores
      uint16_t j[kCap * 64];                   // [position][query] candidate chunks
    } list;
  } w[SelCfg<KQ>::kTiles];
};

}  // namespace

template <int D, int KQ>
__global__ __launch_bounds__(64 * SelCfg<KQ>::kTiles) void select_fast_kernel(const SelectArgs a) {
  constexpr int kTiles = SelCfg<KQ>::kTiles, kCap = SelCfg<KQ>::kCap, kPar = SelCfg<KQ>::kPar;
  constexpr int NS = D / 16;                   // MFMA k-steps over d
  typedef GroupSmem<D, KQ> Smem;
  __shared__ Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int G = (a.N + kTiles - 1) / kTiles;   // tile groups per (batch, head)
  const uint32_t total = (uint32_t)a.B * a.H * G;
  const uint32_t grp = xcd_remap(blockIdx.x, total);
  const int bh = grp / G;
  const int c_top = a.N - 1 - kTiles * (int)(grp % G);   // longest groups first
  // A wave past chunk 0 (N not a multiple of kTiles) runs tile 0 again and writes nothing.
  const bool active = c_top - wave >= 0;
  const int c = max(c_top - wave, 0);
  const int b = bh / a.H, hd = bh % a.H;
  const int n_cand = c + 1;
  const int nb = (n_cand + 31) >> 5;           // this tile's 32-landmark blocks
  const int nbg = (c_top + 1 + 31) >> 5;       // blocks the group sweeps
  const int kq = min(a.k, n_cand);
  const int q0 = c * 64;
  const bf16* Q = static_cast<const bf16*>(a.q) + (size_t)bh * a.L * D;
  const bf16* LM = static_cast<const bf16*>(a.lmk) + (size_t)kv_pair(bh, a.H, a.G) * a.N * D;
  float* ls = &sm.w[wave].list.s[lane];        // this lane's list, stride 64
  uint16_t* lj = &sm.w[wave].list.j[lane];

  // ---------------- q~ as the B operand: query 32 cb + col, d = 16 s + 8 half + z -----------
  bf16x8 qf[2][NS];
  if (a.r > 0) {
    // delta_q^T[d][query] = sum_r W_up[hd*D + d][r] t[query][r]; t (fp32) is split into three
    // bf16 parts so that every product is exact and the sum is accumulated in fp32.
    constexpr int NRS = 4;                     // r <= 64, 16 per step
    const int nrs = (a.r + 15) >> 4;
    bf16x8 tb[3][2][NRS];
    // With r a multiple of 8 every 8-slot run is a whole, 16-byte aligned piece of a row.
    const bool vec = (a.r & 7) == 0;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float* tq = a.tcode + ((size_t)b * a.L + q0 + 32 * cb + col) * a.r;
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        float tv[8];
        if (vec) {
          const int a0 = 16 * rs + 8 * half;
          const f32x4 lo = a0 < a.r ? *reinterpret_cast<const f32x4*>(tq + a0) : zero4();
          const f32x4 hi = a0 < a.r ? *reinterpret_cast<const f32x4*>(tq + a0 + 4) : zero4();
#pragma unroll
          for (int z = 0; z < 4; ++z) {
            tv[z] = lo[z];
            tv[4 + z] = hi[z];
          }
        } else {
#pragma unroll
          for (int z = 0; z < 8; ++z) {
            const int ai = 16 * rs + 8 * half + z;
            tv[z] = (rs < nrs && ai < a.r) ? tq[ai] : 0.f;
          }
        }
#pragma unroll
        for (int z = 0; z < 8; ++z) {
          const float t = tv[z];
          const bf16 t0 = bf16_rne(t);
          const float r1 = t - to_f32(t0);
          const bf16 t1 = bf16_rne(r1);
          tb[0][cb][rs][z] = t0;
          tb[1][cb][rs][z] = t1;
          tb[2][cb][rs][z] = bf16_rne(r1 - to_f32(t1));
        }
      }
    }
    const bf16* WU = static_cast<const bf16*>(a.w_up) + (size_t)hd * D * a.r;
    bf16* qt = sm.w[wave].qt;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      f32x16 acc[2] = {};
      const bf16* wrow = WU + (size_t)(32 * db + col) * a.r;
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        if (rs < nrs) {
          bf16x8 wa;
          if (vec) {
            const int a0 = 16 * rs + 8 * half;
            wa = a0 < a.r ? *reinterpret_cast<const bf16x8*>(wrow + a0) : bf16x8{};
          } else {
#pragma unroll
            for (int z = 0; z < 8; ++z) {
              const int ai = 16 * rs + 8 * half + z;
              wa[z] = ai < a.r ? wrow[ai] : bf16_rne(0.f);
            }
          }
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int p = 0; p < 3; ++p) acc[cb] = mfma32(wa, tb[p][cb][rs], acc[cb]);
        }
      }
      // acc[cb][e]: d = 32 db + 8 (e/4) + 4 half + e%4, query 32 cb + col.
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int qr = 32 * cb + col;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d0 = 32 * db + 8 * a4 + 4 * half;
          const bf16x4 qv = *reinterpret_cast<const bf16x4*>(Q + (size_t)(q0 + qr) * D + d0);
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = bf16_rne(to_f32(qv[i]) + acc[cb][4 * a4 + i]);
          *reinterpret_cast<bf16x4*>(&qt[qr * Smem::QLD + d0]) = o;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        qf[cb][s] = *reinterpret_cast<const bf16x8*>(&qt[(32 * cb + col) * Smem::QLD + 16 * s + 8 * half]);
  } else {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        qf[cb][s] = *reinterpret_cast<const bf16x8*>(Q + (size_t)(q0 + 32 * cb + col) * D + 16 * s + 8 * half);
  }

  // ---------------- landmark ring ------------------------------------------------------------
  // Block jb (landmark rows 32 jb .. 32 jb + 31, clamped to the group's last candidate) is
  // loaded straight into ring slot jb & 1 as NL = 32 * 2D / 1024 loads of 1 KiB, load li by wave
  // li % kTiles; lane l of a load lands at its 1 KiB piece + 16 l.
  auto issue = [&](int jb, int slot) {
    constexpr int VPR = D / 8;                 // 16-byte vectors per row
    constexpr int NL = D / 16;                 // loads per block
    static_assert(NL * 1024 == 32 * Smem::RB, "block size");
#pragma unroll
    for (int li0 = 0; li0 < NL; li0 += kTiles) {
      const int li = li0 + wave;
      if (li < NL) {
        const int r = li * (8 * 64 / D) + lane / VPR, p = lane % VPR;
        const int row = min(32 * jb + r, c_top);
        const bf16* src = LM + (size_t)row * D + 8 * (p ^ ring_swz<D>(r));
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(sm.ring[slot] + 1024 * li), 16, 0, 0);
      }
    }
  };
  // The group walks its blocks in order; f(jb, block) runs once the block is in LDS, while the
  // next block is in flight.  Every wave takes every barrier; f skips blocks past its tile.
  auto sweep = [&](auto&& f) {
    __syncthreads();                           // no wave still reads the ring
    issue(0, 0);
    for (int jb = 0; jb < nbg; ++jb) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();                         // block jb is in LDS; slot (jb + 1) & 1 is free
      if (jb + 1 < nbg) issue(jb + 1, (jb + 1) & 1);
      f(jb, sm.ring[jb & 1]);
    }
  };

  // ---------------- scoring of one 32-landmark block ---------------------------------------
  // A operand: lane (col, half) takes row col, d = 16 s + 8 half .. + 7.  Rows past the last
  // candidate hold later landmarks or repeat the group's last one; their scores are masked.
  auto read_a = [&](const char* blk, bf16x8 (&af)[NS]) {
    const char* rp = blk + col * Smem::RB;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      af[s] = *reinterpret_cast<const bf16x8*>(rp + 16 * ((2 * s + half) ^ ring_swz<D>(col)));
  };
  auto mma_block = [&](const bf16x8 (&af)[NS], f32x16& acc0, f32x16& acc1) {
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
    const int lim = n_cand - 32 * jb;
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
        const int lim = n_cand - 32 * jb;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool out = 8 * (e / 4) + 4 * half + e % 4 >= lim;
          top2(e, out ? -INFINITY : acc0[e]);
          top2(16 + e, out ? -INFINITY : acc1[e]);
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
  int cnt = 0;
  {
    // Make room for the next 8 scores: a list that would overflow is cut to its exact top kq
    // first (rare: lists end near kq + a few).  theta = kq-th largest key, bit by bit from the
    // top, counting list entries in LDS; entries > theta and the first kq - #(> theta)
    // entries == theta stay, in list order.
    auto make_room = [&](const float (&sc)[32], int h0) {
      if (__any(cnt + 8 > kCap)) {
        int np = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) np += sc[h0 + i] >= tau ? 1 : 0;
        if (cnt + np > kCap) {
          // The list's keys in registers (-inf past its end), then theta bit by bit.
          uint32_t key[kCap];
#pragma unroll
          for (int i = 0; i < kCap; ++i) key[i] = f32_key(i < cnt ? ls[64 * i] : -INFINITY);
          uint32_t th = 0u;
          for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = th | (1u << bit);
            int n = 0;
#pragma unroll
            for (int i = 0; i < kCap; ++i) n += key[i] >= cand ? 1 : 0;
            if (n >= kq) th = cand;
          }
          int ngt = 0;
#pragma unroll
          for (int i = 0; i < kCap; ++i) ngt += key[i] > th ? 1 : 0;
          const int m_eq = kq - ngt;
          int w = 0, eq = 0;
#pragma unroll
          for (int i = 0; i < kCap; ++i) {
            bool keep = key[i] > th;
            if (i < cnt && key[i] == th) {
              keep = eq < m_eq;
              ++eq;
            }
            if (keep) {                        // w <= i: entries move towards the front
              const uint16_t jv = lj[64 * i];
              ls[64 * w] = key_f32(key[i]);
              lj[64 * w] = jv;
              ++w;
            }
          }
          cnt = w;
          tau = key_f32(th + 1u);              // later chunks must beat theta strictly
        }
      }
    };
    auto collect = [&](int jb, const float (&sc)[32]) {
#pragma unroll
      for (int h0 = 0; h0 < 32; h0 += 8) {     // at most 8 appends after each check
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
    float sc[32];
    auto keep = [&](int i, float v) { sc[i] = v; };
    sweep([&](int jb, const char* blk) {
      if (jb >= nb) return;
      bf16x8 af[NS];
      read_a(blk, af);
      f32x16 acc0, acc1;
      mma_block(af, acc0, acc1);
      if (jb == nb - 1) for_scores(std::true_type{}, jb, acc0, acc1, keep);
      else for_scores(std::false_type{}, jb, acc0, acc1, keep);
      collect(jb, sc);
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
  const int qpos = q0 + 32 * half + col;
  const size_t orow = ((size_t)bh * a.L + qpos) * a.k;
  int pos = 0;
#pragma unroll
  for (int i = 0; i < kCap; ++i) {
    if (kept[i]) {
      a.idx[orow + pos] = ej[i];
      a.w[orow + pos] = ev[i] * inv;
      ++pos;
    }
  }
  for (int p = kq; p < a.k; ++p) {
    a.idx[orow + p] = -1;
    a.w[orow + p] = 0.f;
  }
}

template <int D>
hipError_t launch_select_fast(const SelectArgs& a, hipStream_t st) {
  if (a.k <= 32) {
    constexpr int T = SelCfg<32>::kTiles;
    const uint32_t groups = (uint32_t)a.B * a.H * ((a.N + T - 1) / T);
    hipLaunchKernelGGL((select_fast_kernel<D, 32>), dim3(groups), dim3(64 * T), 0, st, a);
  } else {
    constexpr int T = SelCfg<64>::kTiles;
    const uint32_t groups = (uint32_t)a.B * a.H * ((a.N + T - 1) / T);
    hipLaunchKernelGGL((select_fast_kernel<D, 64>), dim3(groups), dim3(64 * T), 0, st, a);
  }
  return hipGetLastError();
}

template hipError_t launch_select_fast<64>(const SelectArgs&, hipStream_t);
template hipError_t launch_select_fast<128>(const SelectArgs&, hipStream_t);

}  // namespace hils
