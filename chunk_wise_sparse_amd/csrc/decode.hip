// Decode step: one new token per sequence attends over its key/value cache.
//
// The same method as prefill for a single query at position kv_len-1 (candidates: chunks
// 0..floor((kv_len-1)/C), the last one possibly partial and causally cut at kv_len).  It is
// memory-bound: the step streams every landmark of every (sequence, head) once, then gathers the
// k selected chunks' keys and values once.  Launches on the caller's stream:
//   tcode   - Q-Cal code t_b = W_down h_b per sequence (skipped without Q-Cal);
//   scores  - q~ = round(q + W_up t_b) per workgroup, then the landmark scan, coalesced 16-byte
//             loads, sigma_j = q~ . lmk_j in fp32;
//   select  - exact top-k per (sequence, head) (ties to the smaller chunk index), inter-chunk
//             softmax, ascending output;
//   attend  - per selected chunk: softmax of the raw query over the chunk's visible keys, the
//             weighted partial w_j * o_j in fp32, summed in a fixed order (deterministic): in
//             one workgroup per (sequence, head) when there are enough of them to fill the GPU,
//             else split over workgroups with a separate fixed-order reduction.
// Method: [HiLS-Attention model page, "Model Description"]; [HiLS Attention explainer
// (molayo1419.me), "Core idea" and the Q-Cal item of "Engineering details"]; [news page
// "HiLS Attention Extrapolates 64x ...": per-chunk outputs fused by the retrieval scores].
#include <float.h>

#include "hils_device.h"
#include "hils_launch.h"

namespace hils {

constexpr int kScoreRowsPerWave = 64;                       // landmarks scored by one wave
constexpr int kScoreChunksPerBlock = 4 * kScoreRowsPerWave;   // 4 waves per workgroup

// Lanes sharing one 16-byte-vector row: reduce over the LPR lanes of a row group.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int mk = LPR / 2; mk >= 1; mk >>= 1) v += shfl_xor_f(v, mk);
  return v;
}

// ------------------------------------------------------------------------------------------
// Q-Cal code: t[b][a] = W_down[a] . h_b, one workgroup per (a, b), a fixed summation order.
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void decode_tcode_kernel(const T* __restrict__ hid,
                                                           const T* __restrict__ w_down,
                                                           float* __restrict__ tcode, int D, int r) {
  constexpr int VE = 16 / (int)sizeof(T);
  typedef T vecT __attribute__((ext_vector_type(VE)));
  __shared__ float part[4];
  const int a = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  if (tid == 0) tcode[(size_t)b * r + a] = (part[0] + part[1]) + (part[2] + part[3]);
}

// ------------------------------------------------------------------------------------------
// Landmark scan.
// ------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_scores_kernel(const DecodeArgs a) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int LPR = D / VE;          // lanes per landmark row
  constexpr int RPI = 64 / LPR;        // rows per wave iteration
  constexpr int NIT = kScoreRowsPerWave / RPI;   // iterations for a wave's rows
  typedef T vecT __attribute__((ext_vector_type(VE)));
  __shared__ T qt[D];
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int n_b = (kvl + kChunk - 1) / kChunk;
  const int base = blockIdx.y * kScoreChunksPerBlock + wave * kScoreRowsPerWave;
  if (blockIdx.y * kScoreChunksPerBlock >= n_b) return;   // uniform: the whole workgroup
  const int seg = lane % LPR, sub = lane / LPR;
  const T* L = static_cast<const T*>(a.lmk) + (size_t)bh * a.Nmax * D;
  // Landmark loads first; q~ is formed while they are in flight.
  vecT rows[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = base + it * RPI + sub;
    rows[it] = r < n_b ? *reinterpret_cast<const vecT*>(L + (size_t)r * D + seg * VE) : vecT{};
  }
  // q~[i] = round(q[i] + sum_a W_up[h*D + i][a] t[b][a]) (fp32 sum in order a = 0..r-1; r <= 64).
  for (int i = tid; i < D; i += 256) {
    float dq = 0.f;
    if (a.r > 0) {
      const T* wr = static_cast<const T*>(a.w_up) + ((size_t)h * D + i) * a.r;
      const float* tb = a.tcode + (size_t)b * a.r;
      if (a.r % VE == 0) {                     // rows are 16-byte aligned: vector loads
        vecT wv[64 / VE];
#pragma unroll
        for (int g = 0; g < 64 / VE; ++g)
          if (g * VE < a.r) wv[g] = *reinterpret_cast<const vecT*>(wr + g * VE);
#pragma unroll
        for (int g = 0; g < 64 / VE; ++g)
          if (g * VE < a.r) {
#pragma unroll
            for (int e = 0; e < VE; ++e) dq = fmaf(to_f32(wv[g][e]), tb[g * VE + e], dq);
          }
      } else {
        for (int x = 0; x < a.r; ++x) dq = fmaf(to_f32(wr[x]), tb[x], dq);
      }
    }
    qt[i] = from_f32<T>(to_f32(static_cast<const T*>(a.q)[(size_t)bh * D + i]) + dq);
  }
  __syncthreads();
  const vecT qv = *reinterpret_cast<const vecT*>(&qt[seg * VE]);
  float qf[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) qf[e] = to_f32(qv[e]);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) s = fmaf(to_f32(rows[it][e]), qf[e], s);
    s = row_sum<LPR>(s);
    const int r = base + it * RPI + sub;
    if (seg == 0 && r < n_b) a.scores[(size_t)bh * a.Nmax + r] = s;
  }
}

// Block-wide exclusive scan of one int per thread (256 threads); also returns the total.
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
  for (int w = 0; w < 4; ++w) {
    const int t = scratch[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

// ------------------------------------------------------------------------------------------
// Selection.
// ------------------------------------------------------------------------------------------
// Candidates that fit 32 per thread (n <= 8192): keys in registers, theta (the kk-th largest
// key) by bisection over the key bits with counts from wave ballots, then the selected set as
// bitmaps (chunk order), ties at theta to the smallest indices, and the inter-chunk softmax.
constexpr int kSelReg = 8192;

__global__ __launch_bounds__(256) void decode_select_reg_kernel(const DecodeArgs a) {
  __shared__ float sc[kSelReg];
  __shared__ uint32_t gtw[kSelReg / 32], eqw[kSelReg / 32];
  __shared__ int cnt_w[2][4];
  __shared__ int scratch[8];
  __shared__ uint32_t kmax_w[4];
  __shared__ float evals[64];
  const int bh = blockIdx.x, b = bh / a.H, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
  const int n = (kvl + kChunk - 1) / kChunk;
  const int kk = min(a.k, n);
  const float* G = a.scores + (size_t)bh * a.Nmax;
  uint32_t key[32];
  uint32_t kmax = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int x = tid + 256 * i;
    const float v = x < n ? G[x] : 0.f;
    if (x < n) sc[x] = v;
    key[i] = x < n ? f32_key(v) : 0u;   // 0 is below the key of every finite score
    kmax = max(kmax, key[i]);
  }
#pragma unroll
  for (int mk = 32; mk >= 1; mk >>= 1) kmax = max(kmax, shfl_xor_u(kmax, mk));
  if (lane == 0) kmax_w[wave] = kmax;
  // theta = largest key with #(key >= theta) >= kk, one bit at a time from the top; the wave's
  // count is the popcount of ballots (scalar work), the block's a sum of four slots.
  uint32_t th = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = th | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) c += __popcll(__ballot(key[i] >= cand));
    if (lane == 0) cnt_w[bit & 1][wave] = c;
    __syncthreads();                           // slots alternate, so one barrier per bit
    const int tot = (cnt_w[bit & 1][0] + cnt_w[bit & 1][1]) + (cnt_w[bit & 1][2] + cnt_w[bit & 1][3]);
    if (tot >= kk) th = cand;
  }
  const float smax = key_f32(max(max(kmax_w[0], kmax_w[1]), max(kmax_w[2], kmax_w[3])));
  // Bitmaps of keys > theta and == theta; the wave's 64 lanes cover 64 consecutive chunks.
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint64_t g = __ballot(key[i] > th);
    const uint64_t e = __ballot(key[i] == th);
    if (lane == 0) {
      const int w0 = (256 * i + 64 * wave) >> 5;
      gtw[w0] = (uint32_t)g;
      gtw[w0 + 1] = (uint32_t)(g >> 32);
      eqw[w0] = (uint32_t)e;
      eqw[w0 + 1] = (uint32_t)(e >> 32);
    }
  }
  __syncthreads();
  // Thread t owns chunks 32t .. 32t+31 (ascending).
  const uint32_t gw = gtw[tid], ew = eqw[tid];
  int ngt_total;
  (void)block_exclusive_scan(__popc(gw), scratch, ngt_total);
  const int krem = kk - ngt_total;             // entries == theta to take, smallest first
  int tot;
  const int eq_before = block_exclusive_scan(__popc(ew), scratch, tot);
  const int take = max(0, min(__popc(ew), krem - eq_before));
  uint32_t ek = 0u, rest = ew;
  for (int t = 0; t < take; ++t) {
    ek |= rest & (~rest + 1u);                 // lowest remaining set bit
    rest &= rest - 1u;
  }
  uint32_t sel = gw | ek;
  int pos = block_exclusive_scan(__popc(sel), scratch, tot);
  const float zs = a.scale * 1.4426950408889634f;
  int32_t* I = a.idx + (size_t)bh * a.k;
  float* W = a.w + (size_t)bh * a.k;
  while (sel) {
    const int bt = __builtin_ctz(sel);
    sel &= sel - 1u;
    const int x = 32 * tid + bt;
    I[pos] = x;
    evals[pos] = exp2f((sc[x] - smax) * zs);
    ++pos;
  }
  __syncthreads();
  if (tid < 64) {
    const float e = tid < kk ? evals[tid] : 0.f;
    const float sum = wave_sum(e);
    if (tid < kk) W[tid] = e / sum;
    else if (tid < a.k) { W[tid] = 0.f; I[tid] = -1; }
  }
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
  const int n = (kvl + kChunk - 1) / kChunk;
  const int kk = min(a.k, n);
  const float* G = a.scores + (size_t)bh * a.Nmax;
  auto S = [&](int x) -> float { return G[x]; };

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
// One selected chunk for one wave: softmax of the raw query over the chunk's visible keys and
// the weighted output w_j * o_j (lanes < LPR hold it, VE values each, in acc).
template <typename T, int D>
struct ChunkGather {
  static constexpr int VE = 16 / (int)sizeof(T);
  static constexpr int LPR = D / VE;
  static constexpr int RPI = 64 / LPR;
  static constexpr int NIT = 64 / RPI;
  typedef T vecT __attribute__((ext_vector_type(VE)));
  vecT kr[NIT], vr[NIT];
  int n_vis;
  float wj;

  __device__ __forceinline__ void load(const DecodeArgs& a, int bh, int b, int u, int lane) {
    const int j = u < a.k ? a.idx[(size_t)bh * a.k + u] : -1;
    const int kvl = min(max(a.kv_len[b], 1), a.Lmax);
    const bool live = j >= 0 && j * kChunk < kvl;
    n_vis = live ? min(kChunk, kvl - j * kChunk) : 0;
    wj = live ? a.w[(size_t)bh * a.k + u] : 0.f;
    const int seg = lane % LPR, sub = lane / LPR;
    const size_t row0 = (size_t)bh * a.Lmax + (size_t)(live ? j : 0) * kChunk;
    const T* Kc = static_cast<const T*>(a.k_cache) + row0 * D;
    const T* Vc = static_cast<const T*>(a.v_cache) + row0 * D;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + sub;
      kr[it] = r < n_vis ? *reinterpret_cast<const vecT*>(Kc + (size_t)r * D + seg * VE) : vecT{};
      vr[it] = r < n_vis ? *reinterpret_cast<const vecT*>(Vc + (size_t)r * D + seg * VE) : vecT{};
    }
  }

  // sp: this wave's 64 floats of LDS.  Adds the chunk's weighted output to acc.
  __device__ __forceinline__ void attend(const float (&qf)[VE], float scale, float* sp, int lane,
                                         float (&acc)[VE]) {
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
    __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0): this wave's scores are in LDS
    __builtin_amdgcn_wave_barrier();
    const bool live = n_vis > 0;
    const float zs = scale * 1.4426950408889634f;
    const float sv = sp[lane];
    const float mx = live ? wave_max(sv) : 0.f;
    const float p = live ? exp2f((sv - mx) * zs) : 0.f;
    const float l = wave_sum(p);
    const float f = live ? wj / l : 0.f;
    __builtin_amdgcn_wave_barrier();
    sp[lane] = p * f;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    float part[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) part[e] = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + sub;
      const float pr = sp[r];
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

template <typename T, int D>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int bh, int lane,
                                           float (&qf)[ChunkGather<T, D>::VE]) {
  typedef ChunkGather<T, D> CG;
  const typename CG::vecT qv =
      *reinterpret_cast<const typename CG::vecT*>(static_cast<const T*>(a.q) + (size_t)bh * D + (lane % CG::LPR) * CG::VE);
#pragma unroll
  for (int e = 0; e < CG::VE; ++e) qf[e] = to_f32(qv[e]);
}

// Whole (sequence, head) per workgroup of 8 waves: wave w takes slots w, w + 8, ... in order; the
// 8 wave sums are then added in wave order.  Each wave holds one chunk's keys and values in
// registers (32 KiB for bf16, d = 128), so eight waves keep 256 KiB in flight per workgroup.
template <typename T, int D>
__global__ __launch_bounds__(512) void decode_attend_whole_kernel(const DecodeArgs a) {
  typedef ChunkGather<T, D> CG;
  constexpr int NWV = 8;
  __shared__ float sp[NWV][64];
  __shared__ float wsum[NWV][D];
  const int bh = blockIdx.x, b = bh / a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float qf[CG::VE];
  load_query<T, D>(a, bh, lane, qf);
  float acc[CG::VE];
#pragma unroll
  for (int e = 0; e < CG::VE; ++e) acc[e] = 0.f;
  for (int u = wave; u < a.k; u += NWV) {
    CG cg;
    cg.load(a, bh, b, u, lane);
    cg.attend(qf, a.scale, sp[wave], lane, acc);
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

// Split over workgroups (few (sequence, head) pairs): one wave per slot, partials to memory.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_attend_split_kernel(const DecodeArgs a) {
  typedef ChunkGather<T, D> CG;
  __shared__ float sp[4][64];
  const int bh = blockIdx.x, b = bh / a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int u = blockIdx.y * 4 + wave;
  float qf[CG::VE];
  load_query<T, D>(a, bh, lane, qf);
  float acc[CG::VE];
#pragma unroll
  for (int e = 0; e < CG::VE; ++e) acc[e] = 0.f;
  CG cg;
  cg.load(a, bh, b, u, lane);
  cg.attend(qf, a.scale, sp[wave], lane, acc);
  if (u < a.k && lane < CG::LPR) {
    float* part = a.partial + ((size_t)bh * a.k + u) * D;
#pragma unroll
    for (int e = 0; e < CG::VE; ++e) part[lane * CG::VE + e] = acc[e];
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
    for (int u = gq; u < a.k; u += NG) s += P[(size_t)u * D];
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
  hipLaunchKernelGGL(decode_tcode_kernel<T>, dim3(r, B), dim3(256), 0, st, hid, w_down, tcode, D, r);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t launch_decode_scores(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.B * a.H, (a.Nmax + kScoreChunksPerBlock - 1) / kScoreChunksPerBlock);
  hipLaunchKernelGGL((decode_scores_kernel<T, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_decode_select(const DecodeArgs& a, hipStream_t st) {
  if (a.Nmax <= kSelReg)
    hipLaunchKernelGGL(decode_select_reg_kernel, dim3(a.B * a.H), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(decode_select_kernel, dim3(a.B * a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}
// bf16: whole-pair workgroups once there are at least as many pairs as compute units.
template <typename T, int D>
hipError_t launch_decode_attend(const DecodeArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (a.B * a.H >= 256) {
      hipLaunchKernelGGL((decode_attend_whole_kernel<T, D>), dim3(a.B * a.H), dim3(512), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_attend_split_kernel<T, D>), dim3(a.B * a.H, (a.k + 3) / 4), dim3(256), 0, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(a.B * a.H), dim3(2 * D), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_decode_tcode<bf16>(const bf16*, const bf16*, float*, int, int, int, hipStream_t);
template hipError_t launch_decode_tcode<float>(const float*, const float*, float*, int, int, int, hipStream_t);
#define HILS_DECODE_INST(T, D)                                                      \
  template hipError_t launch_decode_scores<T, D>(const DecodeArgs&, hipStream_t); \
  template hipError_t launch_decode_attend<T, D>(const DecodeArgs&, hipStream_t);
HILS_DECODE_INST(bf16, 64)
HILS_DECODE_INST(bf16, 128)
HILS_DECODE_INST(float, 64)
HILS_DECODE_INST(float, 128)

}  // namespace hils
