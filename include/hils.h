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
 *     synchronised (the one exception: prefill with attn_mode HILS_ATTN_AUTO waits on the stream
 *     once, see there); results are valid once the caller synchronises that stream.
 *   - All checks a host can make run before any launch; on failure nothing is enqueued and a
 *     negative status is returned.  Launch failures return HILS_ERR_HIP; hils_last_hip_error()
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

#define HILS_ABI_VERSION 10

typedef enum {
  HILS_OK = 0,
  HILS_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, aliasing output/input */
  HILS_ERR_UNSUPPORTED = -2,  /* shape or parameter outside what this build supports      */
  HILS_ERR_ALIGNMENT = -3,    /* a pointer is not 16-byte (workspace: 256-byte) aligned   */
  HILS_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required               */
  HILS_ERR_HIP = -5           /* the HIP runtime reported an error                         */
} hils_status;

typedef enum { HILS_DTYPE_BF16 = 0, HILS_DTYPE_FP32 = 1 } hils_dtype;

/* Prefill over a whole sequence.  Supported: head_dim in {64, 128}; chunk in {32, 64, 128};
 * 1 <= topk <= 64; 1 <= seq_len with ceil(seq_len / chunk) <= 65535; 0 <= qcal_rank <= 64;
 * hidden a positive multiple of 128 when qcal_rank > 0.
 * scale <= 0 selects 1/sqrt(head_dim).
 * Chunk sizes 32 and 128, bf16: when seq_len is a multiple of 64, the MFMA selection (64-query
 * tiles scored against their last row's candidates, later landmarks masked per query; the forced
 * local chunk amends it as at chunk 64), else a generic kernel (one query row per wave or per
 * workgroup, scores in LDS); the
 * attention is always the chunk-major MFMA mode (attn_mode and q_tile are ignored, and the
 * workspace is that mode's).  fp32 selects and attends in the generic kernel, whose stage events
 * 2 and 3 are recorded together after it.  Limits: at most 8192 chunks; any seq_len without
 * padding; paged keys/values (pages of chunk rows) for bf16 with seq_len a multiple of the chunk
 * and of 64.  The backward pass takes chunk == 64 only.
 * A partial last chunk (seq_len % chunk != 0) is allowed: lmk then holds ceil(seq_len / chunk)
 * landmarks, the last one for the partial chunk, and the call stages q, k, v, h and o padded to
 * whole chunks in the workspace (the padded rows are zero and come after every real row, so no
 * real row sees them); the stage events then exclude those copies.
 * q_tile: how many consecutive queries share one staged copy of each chunk of their union (the
 *   M adjacent queries of the pages' kernel, HiLS explainer, "Engineering details",
 *   hardware-efficient kernel item): 16, 32, 64 or 128, 0 = 128.  If seq_len is not a multiple,
 *   the largest of these that divides it is used.  It applies to bf16 in the union mode (fp32
 *   keeps a fixed grouping); the results are bitwise the same for every q_tile.
 * stage_events: optional array of n_stage_events hipEvent_t handles (NULL if unused); when it
 * holds at least 4 events, event 0 is recorded before the first kernel and events 1..3 after the
 * Q-Cal, chunk-selection and chunk-attention kernels, on `stream`.
 * attn_mode selects how the chunk attention is organised; both compute the same result:
 *   HILS_ATTN_UNION (0): each group of q_tile consecutive queries stages the union of the chunks
 *     its rows selected, once per group; best when neighbouring rows share most chunks (the
 *     pages report high overlap between adjacent tokens for trained models).
 *   HILS_ATTN_CHUNK_MAJOR (1, bf16 only): per (batch, head) pair the selections are inverted
 *     into per-chunk row lists and each chunk is attended only by the rows that chose it; one
 *     bf16 partial output per (row, slot) in the workspace, summed in slot order.  For
 *     selections with little overlap between neighbouring rows.  The workspace grows by about
 *     seq_len * topk * (2 * head_dim + 4) bytes.
 *   HILS_ATTN_AUTO (2, bf16 only): after the selection, the union size of up to 256 sampled
 *     128-row groups is measured on the GPU and the call waits for it on the host (one stream
 *     synchronisation), then takes the chunk-major mode when the mean union exceeds 8 * topk
 *     chunks (union walk otherwise).  Workspace as for mode 1.  This is the one mode that waits
 *     on the host: on a stream that is being captured it returns HILS_ERR_UNSUPPORTED before
 *     anything is enqueued. */
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
  const int32_t* block_table;  /* device, int32; NULL for contiguous k and v (see below) */
  int32_t block_table_stride;  /* block_table entries per sequence, >= seq_len / chunk */
  int32_t num_pages;           /* pages in the k / v pools when paged */
  int32_t force_local;         /* 1: the query's own chunk is always selected (see below) */
} hils_prefill_params;
/* force_local (prefill and decode; 0 = off, the pages' method): the query's own chunk is always
 * selected, and the other min(k, candidates) - 1 slots hold the best-scoring earlier chunks (ties
 * to the smaller index); the weights stay the softmax over the selection's scores.  Computed by
 * amending the ordinary top-k (a row whose own chunk is missing swaps its worst entry for it),
 * so decode then runs its selection as a separate stage.  The backward pass takes the selection
 * as given and needs no flag. */
/* Paged keys/values (prefill, for a serving cache filled chunk by chunk): with block_table
 * non-NULL, k and v are pools of num_pages pages of one chunk each, [num_pages, kv heads, chunk,
 * head_dim], and chunk j of sequence b is page block_table[b * block_table_stride + j] (entries
 * outside [0, num_pages) are clamped).  q, lmk, h and the outputs keep their layouts.  Needs
 * seq_len a multiple of the chunk (chunks of 32 and 128: bf16 and seq_len also a multiple of
 * 64); the backward pass takes contiguous keys and values only. */

/* One decode step for `batch` sequences, one new token each, at position kv_len[b] - 1 of a
 * key/value cache of capacity max_kv_len (the new token's key and value are already stored).
 * Supported: head_dim in {64, 128}; chunk in {32, 64, 128}; 1 <= topk <= 64;
 * 1 <= max_kv_len <= 65535 * chunk; 0 <= qcal_rank <= 64; hidden a positive multiple of 128
 * when qcal_rank > 0.  A partial last chunk is allowed.  Chunk sizes 32 and 128 take the same
 * landmark scan and selection as 64 and a split attention over C-key chunks (paged caches hold
 * C rows per page; never the one-kernel step below).  With at least 5 stage events, event 0 is
 * recorded first and events 1..4 after the Q-Cal, landmark-scoring, selection and
 * chunk-attention stages; for chunk 64, bf16, batch*heads >= 256 and at most 8192 chunks these
 * three stages run as one kernel, and events 2..4 are recorded together after it. */
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
  int32_t force_local;         /* 1: the query's own chunk is always selected (as prefill) */
} hils_decode_params;
/* Paged caches (decode): with block_table non-NULL, k_cache and v_cache are pools of num_pages
 * pages of one chunk each, [num_pages, kv heads, chunk, head_dim], and chunk j of sequence b is
 * page block_table[b * block_table_stride + j] (entries outside [0, num_pages) are clamped).
 * lmk stays [batch, kv heads, ceil(max_kv_len / chunk), head_dim]. */

/* ABI version this library was built with (HILS_ABI_VERSION). */
int hils_abi_version(void);

/* Workspace bytes needed by one call with these parameters; 0 if the parameters are invalid.
 * with_selection: 1 when the call will pass sel_idx and sel_w (both non-NULL), 0 when both will
 * be NULL.  The selection (chunk indices and weights, [B, H, L, k] each for prefill) is always
 * computed and always read back by the attention stage; when the caller asks for it, the
 * caller's buffers hold it and the workspace leaves it out (at the 128K workload that is 1 GiB
 * less), otherwise the workspace holds it.  The sizes differ by exactly that much. */
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
 *   kv_len    [B] int32, device       valid lengths are 1 <= kv_len[b] <= Lmax.  The host cannot
 *                                     read them; the kernels clamp every value into that range
 *                                     (a value below 1 acts as 1, one above Lmax as Lmax), so an
 *                                     out-of-range length never reads outside the caches.
 *   h         [B, D]; w_down [r, D]; w_up [H*d, r] (NULL iff qcal_rank == 0)
 *   o         [B, H, d]
 *   sel_idx, sel_w [B, H, k]          optional, as for prefill. */
int hils_decode_fwd(const hils_decode_params* p, const void* q, const void* k_cache,
                    const void* v_cache, const void* lmk, const int32_t* kv_len, const void* h,
                    const void* w_down, const void* w_up, void* o, int32_t* sel_idx, float* sel_w,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass of the prefill: gradients of a loss L given dout = dL/do.  The pages learn the
 * chunk selection end to end: the landmark scores sit inside the forward attention, so the loss
 * sends gradients into the landmark keys [HiLS explainer (molayo1419.me), "Core idea: landmark
 * tokens and hierarchical factorisation"; "HiLS Attention Extrapolates 64x at 90% Retrieval
 * Accuracy"].  The forward's selection sel_idx / sel_w ([B, H, L, k], as hils_prefill_fwd
 * returns them) is held fixed: the top-k choice has no gradient.  The rounding of q~ to the run
 * dtype passes gradients unchanged (dq receives both the attention term and the landmark-score
 * term).  Outputs, in the run dtype and the shapes of the matching inputs:
 *   dq [B,H,L,d], dk, dv [B,kv heads,L,d], dlmk [B,kv heads,L/C,d];
 *   with Q-Cal (qcal_rank > 0, else all NULL): dh [B,L,D], dw_down [r,D], dw_up [H*d,r].
 * Every output element is written.  Same shapes and checks as hils_prefill_fwd, plus at most
 * 16384 chunks; q_tile, attn_mode and stage events are ignored.  Sums over rows run in a fixed
 * order: results are bitwise reproducible.  Workspace from hils_prefill_bwd_workspace_size. */
size_t hils_prefill_bwd_workspace_size(const hils_prefill_params* p);
int hils_prefill_bwd(const hils_prefill_params* p, const void* q, const void* k, const void* v, const void* lmk,
                     const void* h, const void* w_down, const void* w_up, const int32_t* sel_idx,
                     const float* sel_w, const void* dout, void* dq, void* dk, void* dv, void* dlmk, void* dh,
                     void* dw_down, void* dw_up, void* workspace, size_t workspace_bytes, void* stream);

/* Dense causal attention: the full-attention baseline the pages compare HiLS with
 * [HiLS explainer (molayo1419.me), "Numerical results": prefill and per-decode-step speed at 512K
 * against full attention on the same hardware].  o_i = sum_t softmax_t(scale q_i . k_t) v_t over
 * every key t <= i (prefill) or over the cache's kv_len[b] keys (decode).  No chunks, no
 * selection.  Same conventions as above (device buffers, stream, checks before any launch,
 * kv_heads for grouped-query attention, clamped kv_len, paged caches not supported).
 * Supported: head_dim in {64, 128}; prefill seq_len a positive multiple of 64.
 * seq_len is the sequence length for prefill and the cache capacity (max_kv_len) for decode. */
typedef struct hils_dense_params {
  int32_t batch, heads, seq_len, head_dim;
  int32_t kv_heads;            /* 0 = heads */
  float scale;                 /* <= 0: 1/sqrt(head_dim) */
  int32_t dtype;               /* hils_dtype */
} hils_dense_params;
/* q [B, H, L, d]; k, v [B, kv heads, L, d]; o [B, H, L, d].  No workspace. */
int hils_dense_prefill_fwd(const hils_dense_params* p, const void* q, const void* k, const void* v, void* o,
                           void* stream);
/* Workspace of one dense decode step: per (sequence, head) the (max, sum, d partial sums) of each
 * span of the cache, fp32; 0 if the parameters are invalid. */
size_t hils_dense_decode_workspace_size(const hils_dense_params* p);
/* q [B, H, d]; k_cache, v_cache [B, kv heads, seq_len, d]; kv_len [B] int32 on the device;
 * o [B, H, d]. */
int hils_dense_decode_fwd(const hils_dense_params* p, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* kv_len, void* o, void* workspace, size_t workspace_bytes, void* stream);

/* HoPE [HiLS explainer (molayo1419.me), "Engineering details", hierarchical positional encoding]:
 * the rotary position encoding on the dimensions inside the pre-training window, none on the
 * others.  Rotates x in place: dimension pair (2i, 2i+1) of a row at position p is turned by the
 * angle p * theta_i, theta_i = rope_base^(-2i / head_dim), when its wavelength 2 pi / theta_i is at
 * most train_len tokens; the other pairs are left as they are.  The caller applies it to q and to
 * k before the attention calls (landmarks and the Q-Cal offset see no position), for decode to
 * the new query and to each key as it enters the cache.
 * x [batch, heads, seq_len, head_dim] on the device, 16-byte aligned (q, or k with heads = the
 * key/value heads).  Row i of sequence b sits at position positions[b] + i when positions (int32
 * [batch], on the device) is given, else at pos0 + i; a decode query takes seq_len = 1 and
 * positions = kv_len - 1.  Angles are reduced modulo 2 pi in fp64, the rotation runs in fp32 and
 * each element is rounded once to the dtype.  Supported: head_dim in {64, 128}; rope_base > 1;
 * train_len >= 1.  Errors as for the other calls; nothing is enqueued on an error. */
typedef struct hils_hope_params {
  int32_t batch, heads, seq_len, head_dim;
  float rope_base;             /* base of the rotary frequencies (for example 10000) */
  int32_t train_len;           /* pre-training window in tokens */
  int32_t pos0;                /* position of row 0 when positions is NULL */
  int32_t dtype;               /* hils_dtype */
} hils_hope_params;
int hils_hope_rotate(const hils_hope_params* p, void* x, const int32_t* positions, void* stream);

/* Landmark of the chunk still being filled during decode.  [HiLS Attention explainer
 * (molayo1419.me), "Core idea: landmark tokens and hierarchical factorisation": a landmark token
 * closes each chunk, so the chunk holding the newest key has none until it has C keys.]  For each
 * sequence b and key/value head g, with n = kv_len[b] clamped to [1, max_kv_len] and
 * j = (n - 1) / chunk, writes lmk[b][g][j] = the mean of k_cache[b][g][j*chunk .. n-1] (fp32 sums
 * in a fixed order, one rounding to the dtype); every other landmark row is left as it is.  The
 * mean is this library's stand-in until the chunk is complete and the model's landmark replaces
 * it; call it after the new key is stored and before hils_decode_fwd.
 * k_cache: [batch, kv_heads, max_kv_len, head_dim], device, read only.  lmk: [batch, kv_heads,
 * ceil(max_kv_len / chunk), head_dim], device, updated in place.  kv_len: [batch] int32, device.
 * Supported: head_dim in {64, 128}; chunk in {32, 64, 128}; dtype bf16 or fp32; contiguous
 * caches (no block table).  Errors as for the other calls; nothing is enqueued on an error. */
typedef struct hils_landmark_params {
  int32_t batch, kv_heads, max_kv_len, head_dim, chunk;
  int32_t dtype;               /* hils_dtype */
} hils_landmark_params;
int hils_partial_landmark(const hils_landmark_params* p, const void* k_cache, void* lmk,
                          const int32_t* kv_len, void* stream);

/* hils_decode_fwd for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops and harnesses that forbid hipMalloc.  The arguments are those of
 * hils_decode_fwd without the workspace; scratch comes from a buffer of
 * HILS_STATIC_SCRATCH_BYTES that the library holds in device memory, one per GPU, from the first
 * call on that GPU (with it current) until the process ends.  The call allocates and frees
 * nothing.  Calls whose hils_decode_workspace_size() exceeds HILS_STATIC_SCRATCH_BYTES return
 * HILS_ERR_WORKSPACE before anything is enqueued (64 MiB covers, for instance, 8 sequences x 32
 * heads at 512K tokens, k = 64, d = 128, which needs about 9 MiB).  Every call on one GPU shares
 * that GPU's buffer: calls that overlap in time on one GPU (two streams, two threads) race and
 * must be serialised by the caller.  No kernel relies on the buffer's contents from an earlier
 * call.  Results are bitwise those of hils_decode_fwd. */
#define HILS_STATIC_SCRATCH_BYTES (64u << 20)
int hils_decode_fwd_noalloc(const hils_decode_params* p, const void* q, const void* k_cache,
                            const void* v_cache, const void* lmk, const int32_t* kv_len, const void* h,
                            const void* w_down, const void* w_up, void* o, int32_t* sel_idx, float* sel_w,
                            void* stream);

/* Static description of a status code. */
const char* hils_status_string(int status);
/* Message of the last failed call on the calling thread: the HIP runtime's error text for
 * HILS_ERR_HIP, or what the validation rejected ("" after a successful call). */
const char* hils_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HILS_H_ */
