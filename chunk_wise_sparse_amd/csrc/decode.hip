// Decode step: one new token per sequence attends over its key/value cache.
//
// The same method as prefill for a single query at position kv_len-1 (candidates: chunks
// 0..floor((kv_len-1)/C), the last one possibly partial and causally cut at kv_len).  It is
// memory-bound: the step streams every landmark of every (sequence, head) once, then gathers the
// k selected chunks' keys and values once.  Launches on the caller's stream:
//   tcode   - Q-Cal code t_b = W_down h_b per sequence (skipped without Q-Cal);
//   fused   - bf16, at least 256 (sequence, head) pairs, up to 8192 chunks: one workgroup per
//             pair forms q~ = round(q + W_up t_b), scores every landmark into LDS, selects the
//             top-k (ties to the smaller chunk index) with the inter-chunk softmax, and gathers
//             the selected chunks.  Otherwise three stages:
//   scores  - q~ per workgroup, then the landmark scan, sigma_j = q~ . lmk_j in fp32; each
//             workgroup keeps its own top-k (up to 8192 chunks) or writes its scores;
//   select  - the exact top-k per (sequence, head), inter-chunk softmax, ascending output;
//   attend  - per selected chunk: softmax of the raw query over the chunk's visible keys, the
//             weighted partial w_j * o_j in fp32, summed in a fixed order (deterministic): in
//             one workgroup per (sequence, head) when there are enough of them to fill the GPU,
//             else split over workgroups with a separate fixed-order reduction.
// Method: [HiLS-Attention model page, "Model Description"]; [HiLS Attention explainer
// (molayo1419.me), "Core idea" and the Q-Cal item of "Engineering details"]; [news page
// "HiLS Attention Extrapolates 64x ...": per-chunk outputs fused by the retrieval scores].
#include <float.h>

#include <algorithm>

#include <type_traits>

#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int kScoreRowsPerWave = 64;                       // landmarks scored by one wave (one per lane)
constexpr int kScoreChunksPerBlock = 4 * kScoreRowsPerWave;   // 4 waves per workgroup
constexpr int kCandSlot = 64;                                // candidates per scan workgroup (k <= 64)

// Lanes sharing one 16-byte-vector row: sum over the LPR lanes of a row group (every lane of the
// group gets it).  Within a 16-lane DPP row the partners come from DPP moves (quad_perm swaps
// of 1 and 2 lanes, then the 8-lane and 16-lane mirrors), wider groups add lane shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row group of 2^n lanes");
  if constexpr (LPR >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if constexpr (LPR >= 16) v += dpp_f<0x140>(v);  // row_mirror
  if constexpr (LPR >= 32) v += shfl_xor_f(v, 16);
  if constexpr (LPR >= 64) v += shfl_xor_f(v, 32);
  return v;
}

// Block-wide exclusive scan of one int per thread (NW waves of 64); also returns the total.
template <int NW = 4>
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
  for (int w = 0; w < NW; ++w) {
    const int t = scratch[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

// Largest t with #(v >= t) >= kk over one wave's NV values per lane (kk >= 1 and at least kk
// values nonzero).
template <int NV>
__device__ __forceinline__ uint32_t wave_kth_key(const uint32_t (&v)[NV], int kk) {
  uint32_t th = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = th | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) c += __popcll(__ballot(v[i] >= cand));
    if (c >= kk) th = cand;
  }
  return th;
}

// ------------------------------------------------------------------------------------------
// Q-Cal code: t[b][a] = W_down[a] . h_b, one workgroup per (a, b), a fixed summation order; rows
// padded with zeros to kTcodeStride entries.
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void decode_tcode_kernel(const T* __restrict__ hid,
                                                           const T* __restrict__ w_down,
                                                           float* __restrict__ tcode, int D, int r) {
  constexpr int VE = 16 / (int)sizeof(T);
  typedef T vecT __attribute__((ext_vector_type(VE)));
  __shared__ float part[4];
  const int a = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a >= r) {                                // padding entries of the row
    if (tid == 0) tcode[(size_t)b * kTcodeStride + a] = 0.f;
    return;
  }
  const T* hb = hid + (size_t)b * D;
  const T* wr = w_down + (size_t)a * D;
  float s = 0.f;
  for (int v = tid; v < D / VE; v += 256) {    // D is a multiple of 128
    const vecT hv = *reinterpret_cast<const vecT*>(hb + (size_t)v * VE);
    const vecT wv = *reinterpret_cast<const vecT*>(wr + (size_t)v * VE);
#pragma unroll
    for (int e = 0; e < VE; ++e) s = fmaf(to_f32(wv[e]), to_f32(hv[e]), s);
  }
  s = wave_sum(s);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  if (tid == 0) tcode[(size_t)b * kTcodeStride + a] = (part[0] + part[1]) + (part[2] + part[3]);
}

// Raw buffer descriptor over `bytes` bytes at p (gfx9 word 3: 32-bit data format).  Every
// operand is wave-uniform; readfirstlane says so to the compiler, since a descriptor lives in
// scalar registers.  Loads through it past `bytes` return zeros without touching memory.
constexpr int kBufDword3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes) {
  const uint64_t base = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), kBufDword3);
}

// ------------------------------------------------------------------------------------------
// Landmark scan.
// ------------------------------------------------------------------------------------------
// kVecW: W_up rows are read as 16-byte vectors (r a nonzero multiple of the vector width).
// Grid (pairs, Y): workgroup y of a pair scores the pair's 256-landmark blocks y, y + Y, ...;
// q~ is formed once per workgroup, while the first block's loads are in flight.
template <typename T, int D, bool kVecW>
__global__ __launch_bounds__(256) void decode_scores_kernel(const DecodeArgs a) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int LPR = D / VE;          // lanes per landmark row
  constexpr int RPI = 64 / LPR;        // rows per load instruction
  constexpr int NIT = kScoreRowsPerWave / RPI;   // load instructions for a wave's rows
  static_assert(D <= 256, "one q~ element per thread");
  typedef T vecT __attribute__((ext_vector_type(VE)));
  __shared__ T qt[256];                        // q~ in entries 0..D-1 (threads >= D write copies)
  __shared__ float tsh[kTcodeStride];          // the sequence's Q-Cal code
  __shared__ float sws[4][4][kScoreRowsPerWave];   // [block q][wave][lane] scores
  __shared__ uint32_t tmx[256];                // candidates: per-thread maximum keys
  __shared__ int wcnt[4][4];                   // candidates per (block, wave); bisection counts
  __shared__ u32x2 clist[4 * kScoreChunksPerBlock];   // candidates in chunk order
  __shared__ u32x2 slot[kCandSlot];            // the workgroup's top-kk
  __shared__ int scratch[4];
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int n_b = (kvl + a.C - 1) / a.C;
  const int nblk = (n_b + kScoreChunksPerBlock - 1) / kScoreChunksPerBlock;
  const int qb = a.score_qb;
  const int blk0 = blockIdx.y * qb;            // this workgroup's blocks: blk0 .. blk0 + nq - 1
  if (blk0 >= nblk) return;                    // uniform: the whole workgroup
  const int nq = min(qb, nblk - blk0);
  int blk = blk0;
  const int seg = lane % LPR, sub = lane / LPR;
  float* S = a.scores + (size_t)bh * a.score_stride;
  // Raw buffer loads through a descriptor over the pair's n_b landmark rows: rows past n_b (and
  // blocks past the last) read as zeros without a memory access, so no load needs a clamp or a
  // branch.
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(static_cast<const T*>(a.lmk) + (size_t)kv_pair(bh, a.H, a.G) * a.Nmax * D,
                                                n_b * D * (int)sizeof(T));
  const int lane_off = (wave * kScoreRowsPerWave * D + sub * D + seg * VE) * (int)sizeof(T);
  constexpr int kBlockBytes = kScoreChunksPerBlock * D * (int)sizeof(T);
  constexpr int kStepBytes = RPI * D * (int)sizeof(T);
  vecT rows[NIT];
  auto load_row = [&](int bk, int it) {
    return __builtin_bit_cast(vecT, __builtin_amdgcn_raw_buffer_load_b128(
                                        rs, bk * kBlockBytes + lane_off + it * kStepBytes, 0, 0));
  };
  // The loads q~ needs are issued first, then the landmark loads; memory counters retire in
  // issue order, so q~ is formed while the landmarks are still in flight.
  const int i = tid % D;                       // q~ element of this thread
  const T* wr = static_cast<const T*>(a.w_up) + ((size_t)h * D + i) * a.r;
  const float qi = to_f32(static_cast<const T*>(a.q)[(size_t)bh * D + i]);
  // The code row is staged in LDS (one load per thread; the row holds kTcodeStride entries).
  const float tv = kVecW ? a.tcode[(size_t)b * kTcodeStride + tid % kTcodeStride] : 0.f;
  vecT wv[64 / VE];
  if constexpr (kVecW) {                       // rows 16-byte aligned, r a multiple of VE
#pragma unroll
    for (int g = 0; g < 64 / VE; ++g)          // group clamped: no branch per load
      wv[g] = *reinterpret_cast<const vecT*>(wr + min(g * VE, a.r - VE));
  }
  asm volatile("" ::: "memory");               // keeps the landmark loads behind these
  // Half of the first block's loads go out before q~ is formed, the rest once its W_up registers
  // are free (fewer registers live at once).
#pragma unroll
  for (int it = 0; it < NIT / 2; ++it) rows[it] = load_row(blk, it);
  // q~[i] = round(q[i] + sum_a W_up[h*D + i][a] t[b][a]) (fp32 sum in order a = 0..r-1; r <= 64).
  {
    float dq = 0.f;
    const float* tb = a.tcode + (size_t)b * kTcodeStride;
    if constexpr (kVecW) {
      static_assert(kTcodeStride == 64, "one W_up row group per 64 code entries");
      if (tid < kTcodeStride) tsh[tid] = tv;
      __syncthreads();
#pragma unroll
      for (int g = 0; g < 64 / VE; ++g) {      // the zero code entries past r add exact zeros
#pragma unroll
        for (int e = 0; e < VE; ++e) dq = fmaf(to_f32(wv[g][e]), tsh[g * VE + e], dq);
      }
    } else {
      for (int x = 0; x < a.r; ++x) dq = fmaf(to_f32(wr[x]), tb[x], dq);
    }
    qt[tid] = from_f32<T>(qi + dq);
  }
#pragma unroll
  for (int it = NIT / 2; it < NIT; ++it) rows[it] = load_row(blk, it);
  __syncthreads();
  const vecT qv = *reinterpret_cast<const vecT*>(&qt[seg * VE]);
  float qf[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) qf[e] = to_f32(qv[e]);
  // Rolling prefetch: once row group it of this block is consumed, its registers take the same
  // row group of the workgroup's next block, so about NIT loads stay in flight per wave (after the
  // last block they address the block past the pair's end: outside the descriptor, no memory
  // traffic).  Scores wait in LDS and leave in one vector store per lane at the end: stores share
  // the vector memory counter with the loads, and every store instruction between the loads
  // holds up the waits on them.
  int q = 0;
  while (true) {
    const int nxt = q + 1 < nq ? blk + 1 : nblk;
    float* sw = sws[q][wave];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) s = fmaf(to_f32(rows[it][e]), qf[e], s);
      rows[it] = load_row(nxt, it);
      s = row_sum<LPR>(s);
      if (seg == 0) sw[it * RPI + sub] = s;
    }
    blk = nxt;
    if (++q >= nq) break;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the wave's scores are in LDS
  __builtin_amdgcn_wave_barrier();
  if (a.cand != nullptr) {
    // Candidates: this workgroup's top-kk chunks under the selection order (score descending,
    // then chunk ascending), kk = min(k, n).  Every chunk of the sequence's top-kk is in the
    // top-kk of its own workgroup, so the workgroups' lists together hold the whole selection.
    // Filter: tau = kk-th largest of the 256 per-thread maxima (at least kk keys reach it, so the
    // local kk-th key does too); the keys >= tau are compacted into LDS in chunk order, and wave 0
    // keeps the exact top-kk among them (all of them when there are too many to rank here).
    const int kk = min(a.k, n_b);
    uint32_t kq[4];
    int xq[4];
    uint32_t m = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xq[q] = (blk0 + q) * kScoreChunksPerBlock + tid;
      kq[q] = (q < nq && xq[q] < n_b) ? f32_key(sws[q][wave][lane]) : 0u;   // 0: no chunk
      m = max(m, kq[q]);
    }
    tmx[tid] = m;
    __syncthreads();
    uint32_t tm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tm[j] = tmx[lane + 64 * j];
    const uint32_t tau = max(wave_kth_key(tm, kk), 1u);   // the same in every wave
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint64_t bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bq[q] = __ballot(kq[q] >= tau);
      if (lane == 0) wcnt[q][wave] = __popcll(bq[q]);
    }
    __syncthreads();
    int run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {              // chunk order: block q, then wave, then lane
      int pre = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int c = wcnt[q][w];
        pre += w < wave ? c : 0;
        tot += c;
      }
      if (kq[q] >= tau) clist[run + pre + __popcll(bq[q] & below)] = u32x2{kq[q], (uint32_t)xq[q]};
      run += tot;
    }
    const int m1 = run;                        // >= 1: the workgroup holds a chunk
    __syncthreads();
    const int kl = min(kk, m1);
    // The exact top-kl of clist under the selection order goes to this workgroup's slot of
    // kCandSlot entries, in chunk order, padded with (0, 0).
    u32x2* out = static_cast<u32x2*>(a.cand) + ((size_t)bh * a.score_ymax + blockIdx.y) * kCandSlot;
    if (m1 <= 256) {
      if (wave != 0) return;
      uint32_t ck[4], cx[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = lane + 64 * j;
        const u32x2 c = clist[min(p, m1 - 1)];
        ck[j] = p < m1 ? c.x : 0u;
        cx[j] = c.y;
      }
      const uint32_t th = wave_kth_key(ck, kl);
      int ngt = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) ngt += __popcll(__ballot(ck[j] > th));
      const int krem = kl - ngt;               // entries at th to keep, earliest chunks first
      int eqb = 0, nout = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool eq = ck[j] == th;
        const uint64_t be = __ballot(eq);
        const bool sel = ck[j] > th || (eq && eqb + __popcll(be & below) < krem);
        eqb += __popcll(be);
        const uint64_t bs = __ballot(sel);
        if (sel) slot[nout + __popcll(bs & below)] = u32x2{ck[j], cx[j]};
        nout += __popcll(bs);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): the slot is in LDS
      __builtin_amdgcn_wave_barrier();
      out[lane] = lane < kl ? slot[lane] : u32x2{0u, 0u};
      return;
    }
    // Many candidates (ties): block-wide.  Thread tid takes entries [tid * P, tid * P + P).
    const int P = (m1 + 255) / 256;            // <= 4
    uint32_t ck[4], cx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid * P + i;
      const u32x2 c = clist[min(p, m1 - 1)];
      ck[i] = (i < P && p < m1) ? c.x : 0u;
      cx[i] = c.y;
    }
    uint32_t th = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = th | (1u << bit);
      int cb = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) cb += __popcll(__ballot(ck[i] >= cand));
      if (lane == 0) wcnt[bit & 1][wave] = cb;
      __syncthreads();                         // slots alternate, so one barrier per bit
      const int tot = (wcnt[bit & 1][0] + wcnt[bit & 1][1]) + (wcnt[bit & 1][2] + wcnt[bit & 1][3]);
      if (tot >= kl) th = cand;
    }
    int ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ngt += ck[i] > th ? 1 : 0;
      neq += ck[i] == th ? 1 : 0;
    }
    int tot, ngt_all;
    (void)block_exclusive_scan(ngt, scratch, ngt_all);
    const int krem = kl - ngt_all;
    int er = block_exclusive_scan(neq, scratch, tot);
    bool sel[4];
    int nsel = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sel[i] = ck[i] > th;
      if (ck[i] == th) { sel[i] = er < krem; ++er; }
      nsel += sel[i] ? 1 : 0;
    }
    int o = block_exclusive_scan(nsel, scratch, tot);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (sel[i]) slot[o++] = u32x2{ck[i], cx[i]};
    __syncthreads();
    if (wave == 0) out[lane] = lane < kl ? slot[lane] : u32x2{0u, 0u};
    return;
  }
  // Thread tid's record: the scores of chunks (blk0 + q) * 256 + tid, q = 0..qb-1 (entries past
  // the sequence's chunks hold values the selection never reads).
  float* rec = S + ((size_t)blockIdx.y * kScoreChunksPerBlock + tid) * qb;
  if (qb == 4) {
    *reinterpret_cast<f32x4*>(rec) = f32x4{sws[0][wave][lane], sws[1][wave][lane], sws[2][wave][lane], sws[3][wave][lane]};
  } else if (qb == 2) {
    *reinterpret_cast<float2*>(rec) = float2{sws[0][wave][lane], sws[1][wave][lane]};
  } else {
    *rec = sws[0][wave][lane];
  }
}

// ------------------------------------------------------------------------------------------
// Selection.
// ------------------------------------------------------------------------------------------
constexpr int kCandCap = 512;                  // candidates the one-wave exact pass takes (8 per lane)

// Candidate slots (n <= 8192): the scan workgroups' top-kk lists, one 64-entry slot each in
// workgroup order, hold the selection's chunks in chunk order; one wave merges them.
struct CandSelSmem {
  float ev[64];
  int32_t sidx[64];                            // the selection, also left in LDS: chunk indices,
  float sw[64];                                // weights (-1 / 0 past kk)
};

// The selection of pair bh by one wave from the scan workgroups' slots (NJ >= the number of
// slots): entry l of slot y sits at list position 64 y + l, and list order is chunk order
// (padding entries have key 0, below every score).  theta, the kk-th largest key, by bisection
// over the key bits; the keys above theta and the earliest entries at theta are kept, in list
// order, with the inter-chunk softmax.  idx / w go to memory and to sm.sidx / sm.sw.
template <int NJ>
__device__ void select_candidates_wave(const DecodeArgs& a, int bh, int kk, int yb, CandSelSmem& sm) {
  const int lane = threadIdx.x & 63;
  const u32x2* L = static_cast<const u32x2*>(a.cand) + (size_t)bh * a.score_ymax * kCandSlot;
  uint32_t ck[NJ], cx[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const u32x2 c = L[min(j, yb - 1) * kCandSlot + lane];
    ck[j] = j < yb ? c.x : 0u;
    cx[j] = c.y;
  }
  uint32_t km = 0u;
#pragma unroll
  for (int j = 0; j < NJ; ++j) km = max(km, ck[j]);
#pragma unroll
  for (int mk = 32; mk >= 1; mk >>= 1) km = max(km, shfl_xor_u(km, mk));
  const float smax = key_f32(km);
  const uint32_t th = wave_kth_key(ck, kk);
  int ngt = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) ngt += __popcll(__ballot(ck[j] > th));
  const int krem = kk - ngt;                   // entries at theta to take, earliest first
  const float zs = a.scale * 1.4426950408889634f;
  int32_t* I = a.idx + (size_t)bh * a.k;
  float* W = a.w + (size_t)bh * a.k;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int eqb = 0, nout = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool eq = ck[j] == th;
    const uint64_t be = __ballot(eq);
    const bool sel = ck[j] > th || (eq && eqb + __popcll(be & below) < krem);
    eqb += __popcll(be);
    const uint64_t bs = __ballot(sel);
    if (sel) {
      const int o = nout + __popcll(bs & below);
      I[o] = (int32_t)cx[j];
      sm.sidx[o] = (int32_t)cx[j];
      sm.ev[o] = exp2f((key_f32(ck[j]) - smax) * zs);
    }
    nout += __popcll(bs);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): ev is in LDS
  __builtin_amdgcn_wave_barrier();
  const float e = lane < kk ? sm.ev[lane] : 0.f;
  const float sum = wave_sum(e);
  const float wv = lane < kk ? e / sum : 0.f;
  if (lane < kk) W[lane] = wv;
  else if (lane < a.k) { W[lane] = 0.f; I[lane] = -1; }
  sm.sw[lane] = wv;
  if (lane >= kk) sm.sidx[lane] = -1;
}

// Wave 0 of the calling workgroup selects for pair bh (the caller synchronises before reading sm).
__device__ __forceinline__ void select_candidates(const DecodeArgs& a, int bh, CandSelSmem& sm) {
  if ((threadIdx.x >> 6) != 0) return;
  const int b = bh / a.H;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int n = (kvl + a.C - 1) / a.C;
  const int kk = min(a.k, n);
  const int yb = ((n + kScoreBlock - 1) / kScoreBlock + a.score_qb - 1) / a.score_qb;   // scan workgroups, <= 32
  if (yb <= 8) select_candidates_wave<8>(a, bh, kk, yb, sm);
  else select_candidates_wave<32>(a, bh, kk, yb, sm);
}

__global__ __launch_bounds__(64) void decode_select_cand_kernel(const DecodeArgs a) {
  __shared__ CandSelSmem sm;
  select_candidates(a, blockIdx.x, sm);
}

// Larger caches: radix select over the scores in global memory, 8 bits at a time.
__global__ __launch_bounds__(256) void decode_select_kernel(const DecodeArgs a) {
  __shared__ int hist[4][256];                 // one histogram per wave, summed in fixed order
  __shared__ int scratch[8];
  __shared__ int bin_found[2];
  __shared__ float evals[64];
  __shared__ uint32_t kmax_w[4];
  const int bh = blockIdx.x, b = bh / a.H, tid = threadIdx.x, wave = tid >> 6;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int n = (kvl + a.C - 1) / a.C;
  const int kk = min(a.k, n);
  const float* G = a.scores + (size_t)bh * a.score_stride;
  auto S = [&](int x) -> float { return G[decode_score_pos(x, a.score_qb)]; };

  // Radix select of the kk-th largest key, 8 bits at a time from the top.
  uint32_t prefix = 0u, pmask = 0u;
  int krem = kk;
  uint32_t kmax = 0u;
  for (int dg = 3; dg >= 0; --dg) {
    for (int x = tid; x < 4 * 256; x += 256) (&hist[0][0])[x] = 0;
    __syncthreads();
    const int sh = dg * 8;
    for (int x = tid; x < n; x += 256) {
      const uint32_t key = f32_key(S(x));
      if (dg == 3) kmax = max(kmax, key);
      if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> sh) & 255u], 1);
    }
    __syncthreads();
    // suffix count for bin tid: sum of hist[tid..255]
    const int bin = 255 - tid;
    const int hv = (hist[0][bin] + hist[1][bin]) + (hist[2][bin] + hist[3][bin]);
    int tot;
    const int ex = block_exclusive_scan(hv, scratch, tot);   // over reversed bins
    const int suffix_incl = ex + hv;                         // bins >= 255 - tid
    const int suffix_excl = ex;                              // bins >  255 - tid
    if (suffix_incl >= krem && suffix_excl < krem) {
      bin_found[0] = bin;
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
  for (int x = lo; x < hi; ++x) eq += f32_key(S(x)) == theta ? 1 : 0;
  int tot;
  int eq_rank = block_exclusive_scan(eq, scratch, tot);
  int nsel = 0;
  {
    int er = eq_rank;
    for (int x = lo; x < hi; ++x) {
      const uint32_t key = f32_key(S(x));
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
      const float sv = S(x);
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

// ------------------------------------------------------------------------------------------
// Chunk attention.
// ------------------------------------------------------------------------------------------
// One selected chunk for one wave.  Rows are read with raw buffer loads through a descriptor
// that covers only the chunk's visible rows: rows past the causal cut (and every row of an empty
// slot) come back as zeros without touching memory, so the loads need no branches and all of a
// chunk's loads are in flight together.
struct Slot {
  int j;        // chunk index, -1 for an empty slot
  int n_vis;    // visible rows (0 for an empty slot)
  float w;      // inter-chunk weight
  int page;     // page of the chunk in a paged cache (0 otherwise)
};

// Page of chunk j of sequence b in a paged cache, clamped to the pool; 0 without a block table.
__device__ __forceinline__ int page_of(const DecodeArgs& a, int b, int j) {
  if (!a.block_table) return 0;
  return min(max(a.block_table[(size_t)b * a.bt_stride + max(j, 0)], 0), a.num_pages - 1);
}

template <typename T, int D>
struct ChunkGather {
  static constexpr int VE = 16 / (int)sizeof(T);
  static constexpr int LPR = D / VE;           // lanes per row
  static constexpr int RPI = 64 / LPR;         // rows per load instruction
  static constexpr int NIT = 64 / RPI;         // load instructions per chunk
  typedef T vecT __attribute__((ext_vector_type(VE)));
  vecT kr[NIT], vr[NIT];

  // Descriptor over the slot's visible rows: in the (sequence, key/value head) cache, or in the
  // slot's page of a paged pool [pages, H/G, 64, d].
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rows(const DecodeArgs& a, const void* cache, int bh,
                                                                const Slot& s) {
    const int kvp = kv_pair(bh, a.H, a.G);
    size_t row0;
    if (a.block_table) {
      const int hk = a.H / a.G;
      row0 = ((size_t)s.page * hk + kvp % hk) * kChunk;
    } else {
      row0 = (size_t)kvp * a.Lmax + (size_t)max(s.j, 0) * kChunk;
    }
    return buffer_rsrc(static_cast<const T*>(cache) + row0 * D, s.n_vis * D * (int)sizeof(T));
  }
  static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, vecT (&dst)[NIT], int lane) {
    const int seg = lane % LPR, sub = lane / LPR;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int off = ((it * RPI + sub) * D + seg * VE) * (int)sizeof(T);
      const u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
      dst[it] = __builtin_bit_cast(vecT, raw);
    }
  }

  // sigma_r = q . k_r for the chunk's rows into this wave's 64 floats of LDS (-inf past n_vis).
  __device__ __forceinline__ void scores(const float (&qf)[VE], int n_vis, float* sp, int lane) const {
    const int seg = lane % LPR, sub = lane / LPR;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) s = fmaf(to_f32(kr[it][e]), qf[e], s);
      s = row_sum<LPR>(s);
      const int r = it * RPI + sub;
      if (seg == 0) sp[r] = r < n_vis ? s : -INFINITY;
    }
  }

  // Softmax over the chunk's scores and the weighted output w_j * o_j added to acc (lanes < LPR
  // hold it, VE values each).
  __device__ __forceinline__ void finish(float scale, const Slot& s, float* sp, int lane,
                                         float (&acc)[VE]) const {
    const int sub = lane / LPR;
    __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0): this wave's scores are in LDS
    __builtin_amdgcn_wave_barrier();
    const bool live = s.n_vis > 0;
    const float zs = scale * 1.4426950408889634f;
    const float sv = sp[lane];
    const float mx = live ? wave_max(sv) : 0.f;
    const float p = live ? exp2f((sv - mx) * zs) : 0.f;
    const float l = wave_sum(p);
    const float f = live ? s.w / l : 0.f;
    __builtin_amdgcn_wave_barrier();
    sp[lane] = p * f;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    float part[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) part[e] = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const float pr = sp[it * RPI + sub];
#pragma unroll
      for (int e = 0; e < VE; ++e) part[e] = fmaf(pr, to_f32(vr[it][e]), part[e]);
    }
#pragma unroll
    for (int mk = LPR; mk < 64; mk <<= 1) {
#pragma unroll
      for (int e = 0; e < VE; ++e) part[e] += shfl_xor_f(part[e], mk);
    }
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] += part[e];
    __builtin_amdgcn_wave_barrier();           // sp is rewritten by the next chunk
  }
};

// Slot u of (sequence b, head): chunk, visible rows and weight.  jl / wl: lane u holds slot u's
// index and weight (lanes >= k: -1 and 0); u is wave-uniform.
__device__ __forceinline__ Slot slot_of(int jl, float wl, int pl, int u, int kvl) {
  Slot s;
  s.j = __builtin_amdgcn_readlane(jl, u);
  s.page = __builtin_amdgcn_readlane(pl, u);
  const bool live = s.j >= 0 && s.j * kChunk < kvl;
  s.n_vis = live ? min(kChunk, kvl - s.j * kChunk) : 0;
  s.w = live ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u)) : 0.f;
  return s;
}

template <typename T, int D>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int bh, int lane,
                                           float (&qf)[ChunkGather<T, D>::VE]) {
  typedef ChunkGather<T, D> CG;
  const typename CG::vecT qv =
      *reinterpret_cast<const typename CG::vecT*>(static_cast<const T*>(a.q) + (size_t)bh * D + (lane % CG::LPR) * CG::VE);
#pragma unroll
  for (int e = 0; e < CG::VE; ++e) qf[e] = to_f32(qv[e]);
}

// Whole (sequence, head) by a workgroup of NWV waves: wave w takes slots w, w + NWV, ... in order;
// the wave sums are then added in wave order.  Each wave holds one chunk's keys and values in
// registers (32 KiB for bf16, d = 128) and keeps the next chunk's loads in flight while it
// computes: the next keys are requested once this chunk's scores are formed, the next values once
// its weighted sum is done.  jl / wl: lane u holds slot u's chunk and weight.
template <typename T, int D, int NWV>
__device__ __forceinline__ void gather_pair(const DecodeArgs& a, int bh, int kvl, int jl, float wl,
                                            float (*sp)[64], float (*wsum)[D]) {
  typedef ChunkGather<T, D> CG;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pl = page_of(a, bh / a.H, jl);     // lane u: page of slot u's chunk (paged caches)
  float qf[CG::VE];
  load_query<T, D>(a, bh, lane, qf);
  float acc[CG::VE];
#pragma unroll
  for (int e = 0; e < CG::VE; ++e) acc[e] = 0.f;
  if (wave < a.k) {
    CG cg;
    int u = wave;
    Slot s = slot_of(jl, wl, pl, u, kvl);
    CG::load(CG::rows(a, a.k_cache, bh, s), cg.kr, lane);
    CG::load(CG::rows(a, a.v_cache, bh, s), cg.vr, lane);
    for (; u + NWV < a.k; u += NWV) {
      cg.scores(qf, s.n_vis, sp[wave], lane);
      const Slot nx = slot_of(jl, wl, pl, u + NWV, kvl);
      CG::load(CG::rows(a, a.k_cache, bh, nx), cg.kr, lane);
      cg.finish(a.scale, s, sp[wave], lane, acc);
      CG::load(CG::rows(a, a.v_cache, bh, nx), cg.vr, lane);
      s = nx;
    }
    cg.scores(qf, s.n_vis, sp[wave], lane);
    cg.finish(a.scale, s, sp[wave], lane, acc);
  }
  if (lane < CG::LPR) {
#pragma unroll
    for (int e = 0; e < CG::VE; ++e) wsum[wave][lane * CG::VE + e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) s += wsum[w][threadIdx.x];
    static_cast<T*>(a.o)[(size_t)bh * D + threadIdx.x] = from_f32<T>(s);
  }
}

// The attention stage alone, one workgroup per (sequence, head).
template <typename T, int D>
__global__ __launch_bounds__(512) void decode_attend_whole_kernel(const DecodeArgs a) {
  typedef ChunkGather<T, D> CG;
  constexpr int NWV = 8;
  __shared__ float sp[NWV][64];
  __shared__ float wsum[NWV][D];
  const int bh = blockIdx.x, b = bh / a.H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  int jl;
  float wl;
  if (a.cand != nullptr && !a.force_local) {   // the selection runs here, from the scan's lists
    __shared__ CandSelSmem sel;
    select_candidates(a, bh, sel);
    __syncthreads();
    jl = lane < a.k ? sel.sidx[lane] : -1;
    wl = lane < a.k ? sel.sw[lane] : 0.f;
  } else {
    jl = lane < a.k ? a.idx[(size_t)bh * a.k + lane] : -1;
    wl = lane < a.k ? a.w[(size_t)bh * a.k + lane] : 0.f;
  }
  gather_pair<T, D, NWV>(a, bh, kvl, jl, wl, sp, wsum);
}

// ------------------------------------------------------------------------------------------
// Fused decode step: one workgroup of 4 waves per (sequence, head) scores the pair's landmarks,
// selects and gathers, with the scores kept in LDS (n <= kFusedMaxChunks).  Used when there are
// at least as many pairs as compute units, so that every compute unit streams its pairs' data
// without a kernel boundary between the stages.
// ------------------------------------------------------------------------------------------
constexpr int kFusedMaxChunks = 8192;
constexpr int kFusedWaves = 4;                 // one wave per SIMD: up to 512 registers each
constexpr int kFusedRowsPerWave = 128;         // landmarks per wave and scan iteration
constexpr int kFusedRows = kFusedWaves * kFusedRowsPerWave;   // per scan iteration (512)

template <typename T, int D, bool kVecW>
__global__ __launch_bounds__(kFusedWaves * 64) void decode_fused_kernel(const DecodeArgs a) {
  constexpr int NWV = kFusedWaves;
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int LPR = D / VE;          // lanes per landmark row
  constexpr int RPI = 64 / LPR;        // rows per load instruction
  constexpr int NIT = kFusedRowsPerWave / RPI;   // load instructions per wave and iteration
  constexpr int NK = kFusedMaxChunks / (NWV * 64);   // keys per thread in the selection (32)
  typedef T vecT __attribute__((ext_vector_type(VE)));
  __shared__ float sc[kFusedMaxChunks];        // the pair's landmark scores
  __shared__ T qt[NWV * 64];                   // q~ in entries 0..D-1 (other threads write copies)
  __shared__ float tsh[kTcodeStride];          // the sequence's Q-Cal code
  __shared__ uint32_t tmx[NWV * 64];           // per-thread maximum keys
  __shared__ int wcnt[2][NK][NWV];             // per (key slot, wave) counts, two uses
  __shared__ int cnt_w[2][NWV];
  __shared__ u32x2 clist[kCandCap];            // candidates in chunk order
  __shared__ CandSelSmem sel;
  __shared__ float sp[NWV][64];
  __shared__ float wsum[NWV][D];
  // With grouped-query heads the G pairs that share a key/value head go to one XCD (one L2), so
  // their landmark and chunk reads are shared there.
  const int bh = a.G > 1 ? (int)xcd_remap(blockIdx.x, gridDim.x) : (int)blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int n = (kvl + kChunk - 1) / kChunk;   // 1 <= n <= kFusedMaxChunks
  const int kk = min(a.k, n);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // ---- landmark scan: iteration it covers rows [512 it, 512 it + 512), wave w 128 of them ----
  const int seg = lane % LPR, sub = lane / LPR;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(static_cast<const T*>(a.lmk) + (size_t)kv_pair(bh, a.H, a.G) * a.Nmax * D,
                                                n * D * (int)sizeof(T));
  const int lane_off = (wave * kFusedRowsPerWave * D + sub * D + seg * VE) * (int)sizeof(T);
  constexpr int kIterBytes = kFusedRows * D * (int)sizeof(T);
  constexpr int kStepBytes = RPI * D * (int)sizeof(T);
  auto load_row = [&](int it, int j) {
    return __builtin_bit_cast(vecT, __builtin_amdgcn_raw_buffer_load_b128(
                                        rs, it * kIterBytes + lane_off + j * kStepBytes, 0, 0));
  };
  const int n_iter = (n + kFusedRows - 1) / kFusedRows;
  // q~ = round(q + W_up[h] t_b): its loads go out first, then half of the first rows; q~ is
  // formed while they are in flight (memory counters retire in issue order).
  const int i = tid % D;
  const T* wr = static_cast<const T*>(a.w_up) + ((size_t)h * D + i) * a.r;
  const float qi = to_f32(static_cast<const T*>(a.q)[(size_t)bh * D + i]);
  const float tv = kVecW ? a.tcode[(size_t)b * kTcodeStride + tid % kTcodeStride] : 0.f;
  vecT wv[64 / VE];
  if constexpr (kVecW) {
#pragma unroll
    for (int g = 0; g < 64 / VE; ++g)          // group clamped: no branch per load
      wv[g] = *reinterpret_cast<const vecT*>(wr + min(g * VE, a.r - VE));
  }
  asm volatile("" ::: "memory");               // keeps the landmark loads behind these
  vecT rows[NIT];
#pragma unroll
  for (int j = 0; j < NIT / 2; ++j) rows[j] = load_row(0, j);
  {
    float dq = 0.f;
    if constexpr (kVecW) {
      if (tid < kTcodeStride) tsh[tid] = tv;
      __syncthreads();
#pragma unroll
      for (int g = 0; g < 64 / VE; ++g)        // the zero code entries past r add exact zeros
#pragma unroll
        for (int e = 0; e < VE; ++e) dq = fmaf(to_f32(wv[g][e]), tsh[g * VE + e], dq);
    } else {
      const float* tb = a.tcode + (size_t)b * kTcodeStride;
      for (int x = 0; x < a.r; ++x) dq = fmaf(to_f32(wr[x]), tb[x], dq);
    }
    qt[tid] = from_f32<T>(qi + dq);
  }
#pragma unroll
  for (int j = NIT / 2; j < NIT; ++j) rows[j] = load_row(0, j);
  __syncthreads();
  float qf[VE];
  {
    const vecT qv = *reinterpret_cast<const vecT*>(&qt[seg * VE]);
#pragma unroll
    for (int e = 0; e < VE; ++e) qf[e] = to_f32(qv[e]);
  }
  // Rolling prefetch: a consumed row group's registers take the same row group of the next
  // iteration (after the last one, rows past n: zeros, no memory traffic).
  for (int it = 0; it < n_iter; ++it) {
    const int nxt = it + 1 < n_iter ? it + 1 : n_iter;
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) s = fmaf(to_f32(rows[j][e]), qf[e], s);
      rows[j] = load_row(nxt, j);
      s = row_sum<LPR>(s);
      if (seg == 0) sc[it * kFusedRows + wave * kFusedRowsPerWave + j * RPI + sub] = s;
    }
  }
  __syncthreads();

  // ---- selection: top-kk under (score descending, chunk ascending) ----
  // Thread tid holds the keys of chunks x = tid + 256 q, q < NK; list order (q, wave, lane) is
  // chunk order.  tau = kk-th largest of the 256 per-thread maxima (every selected key reaches it).
  uint32_t key[NK];
  uint32_t m = 0u;
#pragma unroll
  for (int q = 0; q < NK; ++q) {
    const int x = tid + NWV * 64 * q;
    key[q] = x < n ? f32_key(sc[x]) : 0u;      // 0: no chunk
    m = max(m, key[q]);
  }
  tmx[tid] = m;
  __syncthreads();
  uint32_t tm[NWV];                            // the NWV * 64 maxima, NWV per lane
#pragma unroll
  for (int j = 0; j < NWV; ++j) tm[j] = tmx[lane + 64 * j];
  const uint32_t tau = max(wave_kth_key(tm, kk), 1u);   // the same in every wave
  // Chunk-order positions of the keys >= tau (ballot prefixes and per-(q, wave) counts).
  auto ordered_pos = [&](int use, const bool (&flag)[NK], int (&pos)[NK]) -> int {
    uint64_t bq[NK];
#pragma unroll
    for (int q = 0; q < NK; ++q) {
      bq[q] = __ballot(flag[q]);
      if (lane == 0) wcnt[use][q][wave] = __popcll(bq[q]);
    }
    __syncthreads();
    int run = 0;
#pragma unroll
    for (int q = 0; q < NK; ++q) {
      int pre = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const int c = wcnt[use][q][w];
        pre += w < wave ? c : 0;
        tot += c;
      }
      pos[q] = run + pre + __popcll(bq[q] & below);
      run += tot;
    }
    return run;
  };
  bool fl[NK];
  int pos[NK];
#pragma unroll
  for (int q = 0; q < NK; ++q) fl[q] = key[q] >= tau;
  const int M = ordered_pos(0, fl, pos);       // >= kk
  const float zs = a.scale * 1.4426950408889634f;
  int32_t* I = a.idx + (size_t)bh * a.k;
  float* W = a.w + (size_t)bh * a.k;
  if (M <= kCandCap) {
#pragma unroll
    for (int q = 0; q < NK; ++q)
      if (fl[q]) clist[pos[q]] = u32x2{key[q], (uint32_t)(tid + NWV * 64 * q)};
    __syncthreads();
    // Wave 0 takes the candidates in chunk order, NJ per lane (NJ = 2 covers the usual case of
    // at most 128; the bisection below costs NJ ballots per bit).
    auto exact = [&](auto nj) {
      constexpr int NJ = decltype(nj)::value;
      uint32_t ck[NJ], cx[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int p = lane + 64 * j;
        const u32x2 c = clist[min(p, M - 1)];
        ck[j] = p < M ? c.x : 0u;
        cx[j] = c.y;
      }
      uint32_t km = 0u;
#pragma unroll
      for (int j = 0; j < NJ; ++j) km = max(km, ck[j]);
#pragma unroll
      for (int mk = 32; mk >= 1; mk >>= 1) km = max(km, shfl_xor_u(km, mk));
      const float smax = key_f32(km);
      const uint32_t th = wave_kth_key(ck, kk);
      int ngt = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) ngt += __popcll(__ballot(ck[j] > th));
      const int krem = kk - ngt;               // entries at theta to take, earliest first
      int eqb = 0, nout = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool eq = ck[j] == th;
        const uint64_t be = __ballot(eq);
        const bool s = ck[j] > th || (eq && eqb + __popcll(be & below) < krem);
        eqb += __popcll(be);
        const uint64_t bs = __ballot(s);
        if (s) {
          const int o = nout + __popcll(bs & below);
          sel.sidx[o] = (int32_t)cx[j];
          sel.ev[o] = exp2f((key_f32(ck[j]) - smax) * zs);
        }
        nout += __popcll(bs);
      }
    };
    if (wave == 0) {
      if (M <= 128) exact(std::integral_constant<int, 2>{});
      else exact(std::integral_constant<int, kCandCap / 64>{});
    }
  } else {
    // Many candidates (ties): theta by bisection with block counts, then the keys above theta
    // and the earliest entries at theta, positions in chunk order.
    uint32_t km = 0u;
#pragma unroll
    for (int q = 0; q < NK; ++q) km = max(km, key[q]);
#pragma unroll
    for (int mk = 32; mk >= 1; mk >>= 1) km = max(km, shfl_xor_u(km, mk));
    if (lane == 0) tmx[wave] = km;             // tmx is free again
    uint32_t th = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = th | (1u << bit);
      int cb = 0;
#pragma unroll
      for (int q = 0; q < NK; ++q) cb += __popcll(__ballot(key[q] >= cand));
      if (lane == 0) cnt_w[bit & 1][wave] = cb;
      __syncthreads();                         // slots alternate, so one barrier per bit
      int tot = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) tot += cnt_w[bit & 1][w];
      if (tot >= kk) th = cand;
    }
    uint32_t kmx = 0u;
#pragma unroll
    for (int w = 0; w < NWV; ++w) kmx = max(kmx, tmx[w]);
    const float smax = key_f32(kmx);
    bool gt[NK], eq[NK];
    int epos[NK];
#pragma unroll
    for (int q = 0; q < NK; ++q) {
      gt[q] = key[q] > th;
      eq[q] = key[q] == th;
    }
    const int ngt_all = ordered_pos(1, gt, epos);
    const int krem = kk - ngt_all;
    __syncthreads();                           // wcnt[1] is reused
    (void)ordered_pos(1, eq, epos);            // rank of each entry at theta in chunk order
    bool sl[NK];
#pragma unroll
    for (int q = 0; q < NK; ++q) sl[q] = gt[q] || (eq[q] && epos[q] < krem);
    __syncthreads();
    (void)ordered_pos(1, sl, epos);            // output positions in chunk order
#pragma unroll
    for (int q = 0; q < NK; ++q) {
      if (sl[q]) {
        sel.sidx[epos[q]] = tid + NWV * 64 * q;
        sel.ev[epos[q]] = exp2f((key_f32(key[q]) - smax) * zs);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {                             // weights; idx / w to memory
    const float e = lane < kk ? sel.ev[lane] : 0.f;
    const float sum = wave_sum(e);
    const float wv2 = lane < kk ? e / sum : 0.f;
    const int32_t xi = lane < kk ? sel.sidx[lane] : -1;
    if (lane < a.k) { W[lane] = wv2; I[lane] = xi; }
    sel.sw[lane] = wv2;
    sel.sidx[lane] = xi;
  }
  __syncthreads();

  // ---- chunk attention ----
  const int jl = lane < a.k ? sel.sidx[lane] : -1;
  const float wl = lane < a.k ? sel.sw[lane] : 0.f;
  gather_pair<T, D, NWV>(a, bh, kvl, jl, wl, sp, wsum);
}

// Split over workgroups (few (sequence, head) pairs): one wave per slot, partials to memory.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_attend_split_kernel(const DecodeArgs a) {
  typedef ChunkGather<T, D> CG;
  __shared__ float sp[4][64];
  const int bh = blockIdx.x, b = bh / a.H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u = blockIdx.y * 4 + wave;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  Slot s;
  s.j = u < a.k ? a.idx[(size_t)bh * a.k + u] : -1;
  const bool live = s.j >= 0 && s.j * kChunk < kvl;
  s.n_vis = live ? min(kChunk, kvl - s.j * kChunk) : 0;
  s.w = live ? a.w[(size_t)bh * a.k + u] : 0.f;
  s.page = page_of(a, b, s.j);
  CG cg;
  CG::load(CG::rows(a, a.k_cache, bh, s), cg.kr, lane);
  CG::load(CG::rows(a, a.v_cache, bh, s), cg.vr, lane);
  float qf[CG::VE];
  load_query<T, D>(a, bh, lane, qf);
  float acc[CG::VE];
#pragma unroll
  for (int e = 0; e < CG::VE; ++e) acc[e] = 0.f;
  cg.scores(qf, s.n_vis, sp[wave], lane);
  cg.finish(a.scale, s, sp[wave], lane, acc);
  if (u < a.k && lane < CG::LPR) {
    float* part = a.partial + ((size_t)bh * a.k + u) * D;
#pragma unroll
    for (int e = 0; e < CG::VE; ++e) part[lane * CG::VE + e] = acc[e];
  }
}

// Chunks of C = 32 or 128 keys (contiguous or paged caches): one wave per slot,
// the chunk taken in 64-row pieces (one for C = 32, two for C = 128).  The keys of every piece
// give the chunk's scores, one softmax runs over all of them, then the values of every piece are
// weighted; w_j * o_j goes to the slot's partial as above.  Rows past the chunk's visible ones
// come back as zeros from the buffer loads and score -inf.
template <typename T, int D, int C>
__global__ __launch_bounds__(256) void decode_attend_gc_kernel(const DecodeArgs a) {
  typedef ChunkGather<T, D> CG;
  constexpr int NPC = (C + 63) / 64;           // 64-row pieces of a chunk
  __shared__ float sp[4][NPC * 64];
  const int bh = blockIdx.x, b = bh / a.H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u = blockIdx.y * 4 + wave;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int j = u < a.k ? a.idx[(size_t)bh * a.k + u] : -1;
  const bool live = j >= 0 && j * C < kvl;
  const int n_vis = live ? min(C, kvl - j * C) : 0;
  const float wj = live ? a.w[(size_t)bh * a.k + u] : 0.f;
  // First row of the chunk: in the (sequence, key/value head) cache, or in the chunk's page of a
  // paged pool [pages, H/G, C, d].
  const int kvp = kv_pair(bh, a.H, a.G);
  size_t row0;
  if (a.block_table) {
    const int hk = a.H / a.G;
    row0 = ((size_t)page_of(a, b, j) * hk + kvp % hk) * C;
  } else {
    row0 = (size_t)kvp * a.Lmax + (size_t)max(j, 0) * C;
  }
  auto piece = [&](const void* cache, int pc) {
    const int nv = min(max(n_vis - 64 * pc, 0), 64);
    return buffer_rsrc(static_cast<const T*>(cache) + (row0 + 64 * pc) * D, nv * D * (int)sizeof(T));
  };
  float qf[CG::VE];
  load_query<T, D>(a, bh, lane, qf);
  float* spw = sp[wave];
  CG cg;
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    CG::load(piece(a.k_cache, pc), cg.kr, lane);
    cg.scores(qf, min(max(n_vis - 64 * pc, 0), 64), spw + 64 * pc, lane);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this wave's scores are in LDS
  __builtin_amdgcn_wave_barrier();
  const float zs = a.scale * 1.4426950408889634f;
  float sv[NPC];
  float mx = -INFINITY;
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    sv[pc] = spw[64 * pc + lane];
    mx = fmaxf(mx, sv[pc]);
  }
  mx = live ? wave_max(mx) : 0.f;
  float l = 0.f;
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    sv[pc] = live ? exp2f((sv[pc] - mx) * zs) : 0.f;
    l += sv[pc];
  }
  l = wave_sum(l);
  const float f = live ? wj / l : 0.f;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) spw[64 * pc + lane] = sv[pc] * f;
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  const int sub = lane / CG::LPR;
  float part[CG::VE];
#pragma unroll
  for (int e = 0; e < CG::VE; ++e) part[e] = 0.f;
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    CG::load(piece(a.v_cache, pc), cg.vr, lane);
#pragma unroll
    for (int it = 0; it < CG::NIT; ++it) {
      const float pr = spw[64 * pc + it * CG::RPI + sub];
#pragma unroll
      for (int e = 0; e < CG::VE; ++e) part[e] = fmaf(pr, to_f32(cg.vr[it][e]), part[e]);
    }
  }
#pragma unroll
  for (int mk = CG::LPR; mk < 64; mk <<= 1) {
#pragma unroll
    for (int e = 0; e < CG::VE; ++e) part[e] += shfl_xor_f(part[e], mk);
  }
  if (u < a.k && lane < CG::LPR) {
    float* pt = a.partial + ((size_t)bh * a.k + u) * D;
#pragma unroll
    for (int e = 0; e < CG::VE; ++e) pt[lane * CG::VE + e] = part[e];
  }
}

// o[d] = sum over slots u of partial[u][d] in a fixed order: 8 slot groups (group gq takes
// slots gq, gq + 8, ...), then the groups in order.
template <typename T, int D>
__global__ __launch_bounds__(D * 2) void decode_reduce_kernel(const DecodeArgs a) {
  constexpr int NG = 8;
  __shared__ float part[NG][D];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int d = tid % D, g0 = tid / D;
  const float* P = a.partial + (size_t)bh * a.k * D + d;
#pragma unroll
  for (int gq = g0; gq < NG; gq += 2) {
    float s = 0.f;
    // the group's (at most 8) slots loaded together, then added in slot order
    float pv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int u = gq + NG * t;
      pv[t] = u < a.k ? P[(size_t)u * D] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) s += pv[t];
    part[gq][d] = s;
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int gq = 0; gq < NG; ++gq) s += part[gq][tid];
    static_cast<T*>(a.o)[(size_t)bh * D + tid] = from_f32<T>(s);
  }
}

// ------------------------------------------------------------------------------------------
// Launchers.
// ------------------------------------------------------------------------------------------
template <typename T>
hipError_t launch_decode_tcode(const T* hid, const T* w_down, float* tcode, int B, int D, int r,
                               hipStream_t st) {
  if (r == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_tcode_kernel<T>, dim3(kTcodeStride, B), dim3(256), 0, st, hid, w_down, tcode, D, r);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t launch_decode_scores(const DecodeArgs& a, hipStream_t st) {
  static_assert(kScoreChunksPerBlock == kScoreBlock, "one block = 4 waves x 64 landmarks");
  const int nblk = (a.Nmax + kScoreChunksPerBlock - 1) / kScoreChunksPerBlock;
  dim3 grid(a.B * a.H, (nblk + a.score_qb - 1) / a.score_qb);
  if (a.r > 0 && a.r % (16 / (int)sizeof(T)) == 0)
    hipLaunchKernelGGL((decode_scores_kernel<T, D, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_scores_kernel<T, D, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_decode_select(const DecodeArgs& a, hipStream_t st) {
  if (a.cand != nullptr) {
    hipLaunchKernelGGL(decode_select_cand_kernel, dim3(a.B * a.H), dim3(64), 0, st, a);
  } else {                                     // dense scores (caches of more than 8192 chunks)
    hipLaunchKernelGGL(decode_select_kernel, dim3(a.B * a.H), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}
// bf16: whole-pair workgroups once there are at least as many pairs as compute units; they
// also run the selection when the scan left candidate lists.
template <typename T>
bool decode_attend_whole(const DecodeArgs& a) { return sizeof(T) == 2 && a.B * a.H >= 256; }
template <typename T>
bool decode_select_fused(const DecodeArgs& a) {
  return a.cand != nullptr && !a.force_local && decode_attend_whole<T>(a);
}

// The fused step: bf16, at least as many pairs as compute units, scores that fit in LDS.
template <typename T>
bool decode_fused_ok(const DecodeArgs& a) {
  return sizeof(T) == 2 && a.B * a.H >= 256 && a.Nmax <= kFusedMaxChunks && !a.force_local;
}
template <typename T, int D>
hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t st) {
  if (!decode_fused_ok<T>(a)) return hipErrorInvalidValue;
  if (a.r > 0 && a.r % (16 / (int)sizeof(T)) == 0)
    hipLaunchKernelGGL((decode_fused_kernel<T, D, true>), dim3(a.B * a.H), dim3(kFusedWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL((decode_fused_kernel<T, D, false>), dim3(a.B * a.H), dim3(kFusedWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_attend(const DecodeArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (decode_attend_whole<T>(a)) {
      hipLaunchKernelGGL((decode_attend_whole_kernel<T, D>), dim3(a.B * a.H), dim3(512), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_attend_split_kernel<T, D>), dim3(a.B * a.H, (a.k + 3) / 4), dim3(256), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(a.B * a.H), dim3(2 * D), 0, st, a);
  return hipGetLastError();
}

// Chunks of 32 or 128 keys: the split attention over the selection in idx / w, then the reduce.
template <typename T, int D>
hipError_t launch_decode_attend_gc(const DecodeArgs& a, int C, hipStream_t st) {
  const dim3 grid(a.B * a.H, (a.k + 3) / 4);
  if (C == 32) hipLaunchKernelGGL((decode_attend_gc_kernel<T, D, 32>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((decode_attend_gc_kernel<T, D, 128>), grid, dim3(256), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(a.B * a.H), dim3(2 * D), 0, st, a);
  return hipGetLastError();
}

template bool decode_fused_ok<bf16>(const DecodeArgs&);
template bool decode_fused_ok<float>(const DecodeArgs&);
template bool decode_select_fused<bf16>(const DecodeArgs&);
template bool decode_select_fused<float>(const DecodeArgs&);
template hipError_t launch_decode_tcode<bf16>(const bf16*, const bf16*, float*, int, int, int, hipStream_t);
template hipError_t launch_decode_tcode<float>(const float*, const float*, float*, int, int, int, hipStream_t);
#define HILS_DECODE_INST(T, D)                                                      \
  template hipError_t launch_decode_scores<T, D>(const DecodeArgs&, hipStream_t); \
  template hipError_t launch_decode_fused<T, D>(const DecodeArgs&, hipStream_t); \
  template hipError_t launch_decode_attend<T, D>(const DecodeArgs&, hipStream_t); \
  template hipError_t launch_decode_attend_gc<T, D>(const DecodeArgs&, int, hipStream_t);
HILS_DECODE_INST(bf16, 64)
HILS_DECODE_INST(bf16, 128)
HILS_DECODE_INST(float, 64)
HILS_DECODE_INST(float, 128)

}  // namespace hils
