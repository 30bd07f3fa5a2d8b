// Internal launchers of the HiLS kernels (host side).  Shapes are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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
  int C;                // keys per chunk: 64 (every selection kernel), or 32 / 128 (bf16: the
                        // MFMA selection, L a multiple of 64); N = ceil(L / C)
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
  int q_tile;           // bf16: queries per workgroup (16, 32, 64 or 128), dividing L
  float scale;
  // Paged keys/values (NULL: key / val are [B,H/G,L,d]): key / val are pools of num_pages pages
  // [num_pages, H/G, 64, d] and chunk j of batch b is page block_table[b * bt_stride + j].
  const int32_t* block_table;
  int bt_stride, num_pages;
};

// Chunk-major attention of one (batch, head) pair, bf16: the pair's selections inverted into
// per-chunk lists, each chunk attended only by the rows that selected it (one partial output
// per (row, slot)), then every row's partials summed in slot order.  Pointers are the pair's
// slices; cnt / cur hold N words, off / toff N + 1, ent L * k, partial L * k * d bf16.
struct CmArgs {
  // The batch of (batch, head) pairs pair0 .. pair0 + npairs - 1, one per blockIdx.y of every
  // chunk-major kernel.  Tensors are the whole [B, H, L, ...] (or [B, Hk, L, d]) ones; the list
  // buffers hold npairs consecutive per-pair slices.
  const void* q;        // [B,H,L,d]
  const void* key;      // [B,Hk,L,d] (paged: the pool)
  const void* val;      // [B,Hk,L,d] (paged: the pool)
  const int32_t* idx;   // [B,H,L,k]
  const float* w;       // [B,H,L,k]
  void* o;              // [B,H,L,d]
  uint32_t* cnt;        // [npairs][N] selections per chunk
  uint32_t* off;        // [npairs][N + 1] first list entry of each chunk (exclusive prefix of cnt)
  uint32_t* cur;        // [npairs][N] fill cursors
  uint32_t* toff;       // [npairs][N + 1] first work item of each chunk (prefix of ceil(cnt / kCmItem))
  uint32_t* ent;        // [npairs][L*k][2] list entries (row << 6 | slot, bits of the weight w),
                        // grouped by chunk
  uint32_t* desc;       // [npairs][cm_max_items(L*k, N)][2] work items (first entry, chunk << 8 |
                        // entries), in item order
  void* partial;        // [npairs][L,k,d] bf16: w_j * o_j of slot j of each row
  int L, N, k;
  int C;                // keys per chunk: 64, or 32 / 128 (contiguous keys/values only)
  float scale;
  int H, G, pair0, npairs;   // query heads, query heads per key/value head, the batch of pairs
  // Paged keys/values: key / val are the pools, bt the block table ([B, bt_stride]); NULL: key /
  // val are contiguous [B, Hk, L, d].
  const int32_t* bt;
  int bt_stride, num_pages;
};
constexpr int kCmItem = 128;                   // list entries per work item (8 waves x 16 rows)
// Work items of one pair: each chunk's list is cut into ceil(count / kCmItem) items, so at most
// L*k / kCmItem + N of them.
__host__ __device__ inline size_t cm_max_items(size_t lk, size_t nchunks) { return lk / kCmItem + nchunks + 1; }

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
  int force_local;      // the selection is written out and amended before the attention
  int C;                // keys per chunk: 64; 32 or 128 for the scan, the selection and
                        // launch_decode_attend_gc (pages, if any, hold C rows)
};

// Dense causal attention (the full-attention baseline): prefill over [B,H,L,d] (L % 64 == 0) and
// one decode step over caches [B,H/G,Lmax,d] with per-sequence lengths kv_len.
struct DenseArgs {
  const void* q;        // [B,H,L,d]
  const void* key;      // [B,H/G,L,d]
  const void* val;      // [B,H/G,L,d]
  void* o;              // [B,H,L,d]
  int B, H, L, G;
  float scale;
};
struct DenseDecodeArgs {
  const void* q;        // [B,H,d]
  const void* k_cache;  // [B,H/G,Lmax,d]
  const void* v_cache;
  const int32_t* kv_len;
  float* partial;       // [B*H, splits, d + 2] workspace: (m, l, acc) per span
  void* o;              // [B,H,d]
  int B, H, Lmax, G;
  float scale;
};
template <typename T, int D>
hipError_t launch_dense_prefill(const DenseArgs& a, hipStream_t st);
template <typename T, int D>
hipError_t launch_dense_decode(const DenseDecodeArgs& a, hipStream_t st);
// Spans per (sequence, head) pair of the dense decode step.
int dense_decode_splits(int pairs, int lmax);

// Backward pass of the prefill (the selection held fixed).  Workspace pointers are described
// where they are laid out (hils_api.hip).
struct BwdArgs {
  const void *q, *k_in, *v_in, *lmk, *h, *w_down, *w_up;
  const int32_t* idx;   // [B,H,L,k] the forward's selection
  const float* w;       // [B,H,L,k] the forward's inter-chunk weights
  const void* dout;     // [B,H,L,d]
  void *dq, *dk, *dv, *dlmk, *dh, *dw_down, *dw_up;
  float* tcode;         // [B*L, r] Q-Cal code
  void* qt;             // [B,H,L,d] q~ (run dtype)
  float* dqbuf;         // [B,H,L,d] dq of the chunk attention, then dq~
  float *lse, *dw, *dsig;   // [B,H,L,k] per (row, slot)
  float* dt;            // [B*L, r]
  uint32_t* rbcnt;      // [row blocks, N] counts, then their exclusive prefix per chunk
  uint32_t* choff;      // [N + 1] chunk list offsets
  uint32_t* ent;        // [G*L*k] list entries (g*L + i) << 6 | slot
  float* gpart;         // [splits, max(H*d, hidden), 64] split-K partials
  int B, H, L, G, d, k, r, Dh;
  float scale;
};
template <typename T, int D>
hipError_t launch_prefill_bwd(const BwdArgs& a, hipStream_t st);
size_t bwd_rbcnt_words(int G, int L, int N);
int bwd_splits(int ntok);

// Forced local chunk: after the top-k, rows whose own chunk is not selected swap their worst entry
// for it (see local.hip).  Prefill rows are B*H*L with L the sequence length; decode rows are the
// B*H pairs with L the cache capacity and the query at kv_len[b] - 1.
struct LocalArgs {
  const void* q;        // prefill [B,H,L,d]; decode [B,H,d]
  const void* lmk;      // [B,H/G,N,d]
  const void* w_up;     // [H*d, r]
  const float* tcode;   // Q-Cal code rows, tstride floats apart
  const int32_t* kv_len;   // decode only
  int32_t* idx;         // [rows, k], updated in place
  float* w;             // [rows, k]
  int B, H, L, N, G, k, r, tstride;
  int lc;               // log2 of the chunk size (6: 64 keys)
  float scale;
};
template <typename T, int D>
hipError_t launch_force_local(const LocalArgs& a, bool decode, hipStream_t st);

// nseq sequences of rows (row_bytes each, a multiple of 4) from a rows_src-row layout to a
// rows_dst-row layout: rows past rows_src become zero, rows past rows_dst are dropped.
hipError_t launch_copy_rows(const void* src, void* dst, int nseq, int rows_src, int rows_dst, size_t row_bytes,
                            hipStream_t st);

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
// Chunks of C = 32 or 128 keys (contiguous caches, or pages of C rows; the selection in idx / w):
// split attention into `partial`, then the fixed-order reduce into o.
template <typename T, int D>
hipError_t launch_decode_attend_gc(const DecodeArgs& a, int C, hipStream_t st);

}  // namespace hils
