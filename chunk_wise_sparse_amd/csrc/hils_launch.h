// Internal launchers of the HiLS kernels (host side).  Shapes are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

typedef __bf16 bf16;

struct SelectArgs {
  const void* q;        // [B,H,L,d]
  const void* lmk;      // [B,H/G,N,d]
  const float* tcode;   // [B*L, r] fp32 Q-Cal code (NULL if r == 0)
  const void* w_up;     // [H*d, r]
  int32_t* idx;         // [B,H,L,k]
  float* w;             // [B,H,L,k]
  int B, H, L, N, k, r;
  int G;                // query heads per key/value (and landmark) head
  float scale;
};

struct AttnArgs {
  const void* q;        // [B,H,L,d]
  const void* key;      // [B,H/G,L,d]
  const void* val;      // [B,H/G,L,d]
  const int32_t* idx;   // [B,H,L,k]
  const float* w;       // [B,H,L,k]
  void* o;              // [B,H,L,d]
  int B, H, L, N, topk;
  int G;                // query heads per key/value head
  float scale;
};

// Chunk-major attention of one (batch, head) pair, bf16: the pair's selections inverted into
// per-chunk lists, each chunk attended only by the rows that selected it (one partial output
// per (row, slot)), then every row's partials summed in slot order.  Pointers are the pair's
// slices; cnt / cur hold N words, off / toff N + 1, ent L * k, partial L * k * d bf16.
struct CmArgs {
  const void* q;        // [L,d]
  const void* key;      // [L,d]
  const void* val;      // [L,d]
  const int32_t* idx;   // [L,k]
  const float* w;       // [L,k]
  void* o;              // [L,d]
  uint32_t* cnt;        // selections per chunk
  uint32_t* off;        // first list entry of each chunk (exclusive prefix of cnt)
  uint32_t* cur;        // fill cursors
  uint32_t* toff;       // first work item of each chunk (prefix of ceil(cnt / kCmItem))
  uint32_t* ent;        // list entries (row << 6 | slot), grouped by chunk
  void* partial;        // [L,k,d] bf16: w_j * o_j of slot j of each row
  int L, N, k;
  float scale;
};
constexpr int kCmItem = 128;                   // list entries per work item (8 waves x 16 rows)

// Decode Q-Cal code rows are padded to this many entries (zeros past the rank).
constexpr int kTcodeStride = 64;

// Decode landmark scores are stored workgroup-major.  The scan workgroup (pair, y) scores the qb
// consecutive 256-landmark blocks y*qb .. y*qb+qb-1, and its thread t keeps the qb scores of
// chunks (y*qb+q)*256 + t, q = 0..qb-1, side by side: one vector store per wave writes them.
// qb is 4, 2 or 1, the largest that still gives the scan about 1024 workgroups.
constexpr int kScoreBlock = 256;               // landmarks per block (4 waves x 64)
inline int decode_score_qb(int pairs, int nmax) {
  const int nblk = (nmax + kScoreBlock - 1) / kScoreBlock;
  for (int qb = 4; qb > 1; qb >>= 1)
    if ((long long)pairs * ((nblk + qb - 1) / qb) >= 1024) return qb;
  return 1;
}
// Floats per pair of the score buffer.
inline size_t decode_score_stride(int nmax, int qb) {
  const int nblk = (nmax + kScoreBlock - 1) / kScoreBlock;
  return (size_t)((nblk + qb - 1) / qb) * qb * kScoreBlock;
}
// Position of chunk x's score in its pair's part of the buffer.
__host__ __device__ inline int decode_score_pos(int x, int qb) {
  const int b = x / kScoreBlock;
  return ((b / qb) * kScoreBlock + x % kScoreBlock) * qb + b % qb;
}

struct DecodeArgs {
  const void* q;        // [B,H,d] raw query
  const void* w_up;     // [H*d, r] Q-Cal up-projection (unused when r == 0)
  const float* tcode;   // [B, kTcodeStride] Q-Cal code W_down h, zero past r (workspace)
  const void* k_cache;  // [B,H/G,Lmax,d]
  const void* v_cache;
  const void* lmk;      // [B,H/G,Nmax,d]
  const int32_t* kv_len;
  float* scores;        // [B*H][score_stride] workspace, workgroup-major (decode_score_pos)
  int32_t* idx;         // [B,H,k]
  float* w;             // [B,H,k]
  float* partial;       // [B,H,k,d] workspace (split attend only)
  void* o;              // [B,H,d]
  int B, H, Lmax, Nmax, k, r;
  int G;                // query heads per key/value (and landmark) head
  // Paged caches (NULL: k_cache / v_cache are [B,H/G,Lmax,d]): k_cache / v_cache are pools of
  // num_pages pages [num_pages, H/G, 64, d], and chunk j of sequence b is page
  // block_table[b * bt_stride + j] (clamped to the pool).
  const int32_t* block_table;
  int bt_stride, num_pages;
  int score_qb;         // decode_score_qb(B*H, Nmax)
  size_t score_stride;  // decode_score_stride(Nmax, score_qb)
  // Candidate mode (Nmax <= 8192; NULL otherwise): scan workgroup (pair, y) writes its top-k
  // (key, chunk) pairs in chunk order to the 64-entry slot cand[(pair * score_ymax + y) * 64],
  // padded with (0, 0); no dense scores are written.
  void* cand;           // uint32 pairs (key, chunk)
  int score_ymax;       // scan workgroups per pair: ceil(ceil(Nmax / 256) / score_qb)
  float scale;
};

template <typename T>
hipError_t launch_prefill_qcal_code(const T* h, const T* w_down, float* t_out, int n_tok, int D,
                                    int r, hipStream_t st);

template <typename T, int D>
hipError_t launch_select(const SelectArgs& a, hipStream_t st);
template <int D>
hipError_t launch_select_fast(const SelectArgs& a, hipStream_t st);   // bf16, k <= 64
template <typename T, int D>
hipError_t launch_chunk_attention(const AttnArgs& a, hipStream_t st);
template <int D>
hipError_t launch_chunk_attention_cm(const CmArgs& a, hipStream_t st);
// Sum over up to 256 sampled 128-row groups of the number of distinct chunks their rows selected
// (one uint32 at *total, overwritten); the number of groups sampled is returned in *groups.
hipError_t launch_union_probe(const int32_t* idx, int B, int H, int L, int k, uint32_t* total,
                              int* groups, hipStream_t st);

template <typename T>
hipError_t launch_decode_tcode(const T* hid, const T* w_down, float* tcode, int B, int D, int r,
                               hipStream_t st);
template <typename T, int D>
hipError_t launch_decode_scores(const DecodeArgs& a, hipStream_t st);
// The whole step after the Q-Cal code in one kernel (one workgroup per (sequence, head)); only
// when decode_fused_ok<T>(a).
template <typename T>
bool decode_fused_ok(const DecodeArgs& a);
template <typename T, int D>
hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_select(const DecodeArgs& a, hipStream_t st);
// True when launch_decode_attend<T, D> performs the selection itself (launch_decode_select is
// then skipped).
template <typename T>
bool decode_select_fused(const DecodeArgs& a);
template <typename T, int D>
hipError_t launch_decode_attend(const DecodeArgs& a, hipStream_t st);

}  // namespace hils
