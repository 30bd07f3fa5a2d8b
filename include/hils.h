/* hils.h — C ABI of the HiLS (Hierarchical Landmark Sparse) attention forward pass on AMD MI355X.
 *
 * What the two entry points compute, per query row (batch b, head h, position i):
 *   1. Q-Cal: q~ = round_dtype(q + W_up[h] (W_down h_i)), a low-rank offset of the query that is
 *      used only to score chunks.  [HiLS Attention explainer (molayo1419.me), "Engineering
 *      details", Q-Cal item.]
 *   2. Inter-chunk scores: sigma_j = q~ . lmk_j over the causal chunks j <= floor(i / C), the
 *      query's own chunk included; lmk_j is the landmark key of chunk j.  [HiLS-Attention model
 *      page, "Model Description"; explainer, "Core idea", level 1.]
 *   3. Top-k: the k largest sigma (ties to the smaller chunk index); fewer than k candidates
 *      select them all.  [Model page: the top-k chunks are selected.]
 *   4. Inter-chunk softmax: w_j = softmax over the selection of scale * sigma_j.  [Model page:
 *      attention factorised into an inter-chunk and an intra-chunk softmax.]
 *   5. Intra-chunk attention of the raw q over each selected chunk's keys/values, the own chunk
 *      causally truncated at i: o_j = softmax_t(scale * q . k_t) V.  [Explainer, "Core idea",
 *      level 2; "HiLS Attention Extrapolates 64x at 90% Retrieval Accuracy": each chunk is
 *      attended independently.]
 *   6. Fusion: o = sum_j w_j o_j.  [Same news page: outputs fused by the retrieval scores.]
 *
 * Conventions for every call:
 *   - Tensors are device memory, contiguous row-major, 16-byte aligned, element type `dtype`
 *     unless stated.  The caller owns every buffer; the library keeps no pointer after the call.
 *   - Inputs are read-only.  Every output element is written (idx padding -1, w padding 0).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and nothing is
 *     synchronised; results are valid once the caller synchronises that stream.
 *   - All checks a host can make run before any launch; on failure nothing is enqueued and a
 *     negative status is returned.  Launch failures return HILS_ERR_HIP; hils_last_error()
 *     gives the message (per thread).
 *   - The library allocates no device memory.  Scratch comes from the caller's workspace, of
 *     at least *_workspace_size() bytes, 256-byte aligned.
 *   - Results are bitwise reproducible for identical inputs and launch parameters.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef HILS_H_
#define HILS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HILS_ABI_VERSION 5

typedef enum {
  HILS_OK = 0,
  HILS_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, aliasing output/input */
  HILS_ERR_UNSUPPORTED = -2,  /* shape or parameter outside what this build supports      */
  HILS_ERR_ALIGNMENT = -3,    /* a pointer is not 16-byte (workspace: 256-byte) aligned   */
  HILS_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required               */
  HILS_ERR_HIP = -5           /* the HIP runtime reported an error                         */
} hils_status;

typedef enum { HILS_DTYPE_BF16 = 0, HILS_DTYPE_FP32 = 1 } hils_dtype;

/* Prefill over a whole sequence.  Supported: head_dim in {64, 128}; chunk == 64;
 * 1 <= topk <= 64; seq_len a positive multiple of chunk with seq_len / chunk <= 65535
 * (<= 16384 for fp32 with head_dim 128); q_tile == 64 (or 0 for the default);
 * 0 <= qcal_rank <= 64; hidden a positive multiple of 128 when qcal_rank > 0.  scale <= 0 selects 1/sqrt(head_dim).
 * stage_events: optional array of n_stage_events hipEvent_t handles (NULL if unused); when it
 * holds at least 4 events, event 0 is recorded before the first kernel and events 1..3 after the
 * Q-Cal, chunk-selection and chunk-attention kernels, on `stream`.
 * attn_mode selects how the chunk attention is organised; both compute the same result:
 *   HILS_ATTN_UNION (0): each group of 128 consecutive queries stages the union of the chunks
 *     its rows selected, once per group; best when neighbouring rows share most chunks (the
 *     pages report high overlap between adjacent tokens for trained models).
 *   HILS_ATTN_CHUNK_MAJOR (1, bf16 only): per (batch, head) pair the selections are inverted
 *     into per-chunk row lists and each chunk is attended only by the rows that chose it; one
 *     bf16 partial output per (row, slot) in the workspace, summed in slot order.  For
 *     selections with little overlap between neighbouring rows.  The workspace grows by about
 *     seq_len * topk * (2 * head_dim + 4) bytes.
 *   HILS_ATTN_AUTO (2, bf16 only): after the selection, the union size of up to 256 sampled
 *     128-row groups is measured on the GPU and the call waits for it on the host (one stream
 *     synchronisation, so not for graph capture), then takes the chunk-major mode when the mean
 *     union exceeds 8 * topk chunks (union walk otherwise).  Workspace as for mode 1. */
typedef enum { HILS_ATTN_UNION = 0, HILS_ATTN_CHUNK_MAJOR = 1, HILS_ATTN_AUTO = 2 } hils_attn_mode;
/* Grouped-query attention (both calls): kv_heads > 0 must divide heads; query head h then uses
 * key/value head h / (heads / kv_heads), and k, v, lmk (prefill) or k_cache, v_cache, lmk
 * (decode) hold kv_heads heads instead of heads.  Landmarks belong to the key/value head.
 * Selection, weights and outputs stay per query head.  kv_heads = 0 or heads: one key/value
 * head per query head. */
typedef struct hils_prefill_params {
  int32_t batch, heads, seq_len, head_dim;
  int32_t chunk, topk, q_tile;
  int32_t hidden, qcal_rank;
  float scale;
  int32_t dtype;               /* hils_dtype */
  void* const* stage_events;
  int32_t n_stage_events;
  int32_t attn_mode;           /* hils_attn_mode */
  int32_t kv_heads;            /* key/value (and landmark) heads; 0 = heads (see below) */
} hils_prefill_params;

/* One decode step for `batch` sequences, one new token each, at position kv_len[b] - 1 of a
 * key/value cache of capacity max_kv_len (the new token's key and value are already stored).
 * Supported: head_dim in {64, 128}; chunk == 64; 1 <= topk <= 64;
 * 1 <= max_kv_len <= 65535 * chunk; 0 <= qcal_rank <= 64; hidden a positive multiple of 128
 * when qcal_rank > 0.  A partial last chunk is allowed.  With at least 5 stage events, event 0 is
 * recorded first and events 1..4 after the Q-Cal, landmark-scoring, selection and
 * chunk-attention stages; for bf16 with batch*heads >= 256 and at most 8192 chunks these three
 * stages run as one kernel, and events 2..4 are recorded together after it. */
typedef struct hils_decode_params {
  int32_t batch, heads, max_kv_len, head_dim;
  int32_t chunk, topk;
  int32_t hidden, qcal_rank;
  float scale;
  int32_t dtype;
  void* const* stage_events;
  int32_t n_stage_events;
  int32_t kv_heads;            /* key/value (and landmark) heads; 0 = heads (see below) */
  const int32_t* block_table;  /* device, int32; NULL for contiguous caches (see below) */
  int32_t block_table_stride;  /* block_table entries per sequence, >= ceil(max_kv_len / chunk) */
  int32_t num_pages;           /* pages in the k_cache / v_cache pools when paged */
} hils_decode_params;
/* Paged caches (decode): with block_table non-NULL, k_cache and v_cache are pools of num_pages
 * pages of one chunk each, [num_pages, kv heads, chunk, head_dim], and chunk j of sequence b is
 * page block_table[b * block_table_stride + j] (entries outside [0, num_pages) are clamped).
 * lmk stays [batch, kv heads, ceil(max_kv_len / chunk), head_dim]. */

/* ABI version this library was built with (HILS_ABI_VERSION). */
int hils_abi_version(void);

/* Workspace bytes needed by one call with these parameters; 0 if the parameters are invalid.
 * The size depends on whether sel_idx / sel_w will be passed (if both are given they double as
 * scratch and the workspace shrinks): pass with_selection = 1 when both will be non-NULL. */
size_t hils_prefill_workspace_size(const hils_prefill_params* p, int with_selection);
size_t hils_decode_workspace_size(const hils_decode_params* p, int with_selection);

/* Prefill.
 *   q, k, v   [B, H, L, d]            queries, keys, values (q raw, before Q-Cal)
 *   lmk       [B, H, L / C, d]        one landmark key per chunk
 *   h         [B, L, D]               hidden states for Q-Cal (NULL iff qcal_rank == 0)
 *   w_down    [r, D], w_up [H*d, r]   Q-Cal factors (NULL iff qcal_rank == 0)
 *   o         [B, H, L, d]            output
 *   sel_idx   [B, H, L, k] int32      selected chunks, ascending, -1 padded (NULL: not returned)
 *   sel_w     [B, H, L, k] float32    inter-chunk weights, 0 padded (NULL: not returned)
 * sel_idx and sel_w must be both NULL or both non-NULL. */
int hils_prefill_fwd(const hils_prefill_params* p, const void* q, const void* k, const void* v,
                     const void* lmk, const void* h, const void* w_down, const void* w_up, void* o,
                     int32_t* sel_idx, float* sel_w, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Decode.
 *   q         [B, H, d]               the new token's raw query
 *   k_cache, v_cache [B, H, Lmax, d]  caches; rows >= kv_len[b] are never read
 *   lmk       [B, H, ceil(Lmax / C), d] landmark keys (chunks at or beyond kv_len are ignored)
 *   kv_len    [B] int32, device       1 <= kv_len[b] <= Lmax (not checked on the host: values
 *                                     outside that range are undefined behaviour)
 *   h         [B, D]; w_down [r, D]; w_up [H*d, r] (NULL iff qcal_rank == 0)
 *   o         [B, H, d]
 *   sel_idx, sel_w [B, H, k]          optional, as for prefill. */
int hils_decode_fwd(const hils_decode_params* p, const void* q, const void* k_cache,
                    const void* v_cache, const void* lmk, const int32_t* kv_len, const void* h,
                    const void* w_down, const void* w_up, void* o, int32_t* sel_idx, float* sel_w,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* hils_status_string(int status);
/* Message of the last HILS_ERR_HIP / validation failure on the calling thread ("" if none). */
const char* hils_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HILS_H_ */
