// C ABI of the HiLS forward pass: argument validation, workspace layout and launch sequencing.
// Every host-checkable error is reported before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "hils.h"
#include "hils_launch.h"
#include "gchunk.h"
#include "landmark.h"
#include "hope.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(HILS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kWsAlign = 256;
size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};
bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

size_t elem_bytes(int dtype) { return dtype == HILS_DTYPE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------------------------
struct PrefillLayout {
  size_t tcode, idx, w, probe, cm_cnt, cm_off, cm_cur, cm_toff, cm_ent, cm_desc, cm_partial, total;
};

int check_prefill_params(const hils_prefill_params* p) {
  if (!p) return fail(HILS_ERR_INVALID_ARG, "params is NULL");
  if (p->batch <= 0 || p->heads <= 0 || p->seq_len <= 0 || p->head_dim <= 0)
    return fail(HILS_ERR_INVALID_ARG, "batch, heads, seq_len and head_dim must be positive");
  if (p->dtype != HILS_DTYPE_BF16 && p->dtype != HILS_DTYPE_FP32)
    return fail(HILS_ERR_UNSUPPORTED, "dtype %d is not supported", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HILS_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", p->head_dim);
  if (p->chunk != 64 && p->chunk != 32 && p->chunk != 128)
    return fail(HILS_ERR_UNSUPPORTED, "chunk %d is not supported (32, 64 or 128)", p->chunk);
  if (p->topk < 1 || p->topk > 64)
    return fail(HILS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", p->topk);
  if ((p->seq_len + 63) / 64 > 65535)
    return fail(HILS_ERR_UNSUPPORTED, "more than 65535 chunks per sequence");
  if (p->chunk != 64) {
    if ((p->seq_len + p->chunk - 1) / p->chunk > hils::kGcMaxChunks)
      return fail(HILS_ERR_UNSUPPORTED, "chunk %d: at most %d chunks per sequence", p->chunk, hils::kGcMaxChunks);
    if (p->block_table && (p->dtype != HILS_DTYPE_BF16 || p->seq_len % 64 != 0))
      return fail(HILS_ERR_UNSUPPORTED, "chunk %d: paged keys/values need bf16 and seq_len a multiple of 64",
                  p->chunk);
  }
  if (p->q_tile != 0 && p->q_tile != 16 && p->q_tile != 32 && p->q_tile != 64 && p->q_tile != 128)
    return fail(HILS_ERR_UNSUPPORTED, "q_tile %d is not supported (16, 32, 64 or 128)", p->q_tile);
  if (p->qcal_rank < 0 || p->qcal_rank > 64)
    return fail(HILS_ERR_UNSUPPORTED, "qcal_rank %d outside [0, 64]", p->qcal_rank);
  if (p->qcal_rank > 0 && (p->hidden <= 0 || p->hidden % 128 != 0))
    return fail(HILS_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 128", p->hidden);
  if (!(isfinite(p->scale))) return fail(HILS_ERR_INVALID_ARG, "scale is not finite");
  if (p->n_stage_events < 0 || (p->n_stage_events > 0 && !p->stage_events))
    return fail(HILS_ERR_INVALID_ARG, "stage_events inconsistent with n_stage_events");
  if (p->kv_heads < 0 || p->kv_heads > p->heads || (p->kv_heads > 0 && p->heads % p->kv_heads != 0))
    return fail(HILS_ERR_INVALID_ARG, "kv_heads %d must divide heads %d", p->kv_heads, p->heads);
  if (p->attn_mode != HILS_ATTN_UNION && p->attn_mode != HILS_ATTN_CHUNK_MAJOR && p->attn_mode != HILS_ATTN_AUTO)
    return fail(HILS_ERR_UNSUPPORTED, "attn_mode %d is not supported", p->attn_mode);
  if (p->attn_mode != HILS_ATTN_UNION && p->dtype != HILS_DTYPE_BF16)
    return fail(HILS_ERR_UNSUPPORTED, "the chunk-major attention mode is bf16 only");
  if (p->force_local != 0 && p->force_local != 1)
    return fail(HILS_ERR_INVALID_ARG, "force_local must be 0 or 1");
  if (p->block_table) {
    if (p->seq_len % p->chunk != 0)
      return fail(HILS_ERR_UNSUPPORTED, "paged keys/values need seq_len a multiple of the chunk (%d)", p->chunk);
    if (p->num_pages < 1 || p->block_table_stride < p->seq_len / p->chunk)
      return fail(HILS_ERR_INVALID_ARG, "paged keys/values: num_pages >= 1 and block_table_stride >= %d needed",
                  p->seq_len / p->chunk);
    if ((uintptr_t)p->block_table & 3) return fail(HILS_ERR_ALIGNMENT, "block_table is not 4-byte aligned");
  }
  const double bhld = (double)p->batch * p->heads * (p->seq_len + 63.0) * p->head_dim;
  if (bhld > 4e18 / 8 || (double)p->batch * p->heads * ((p->seq_len + 63) / 64) > 2147483647.0)
    return fail(HILS_ERR_UNSUPPORTED, "problem too large");
  return HILS_OK;
}

// Queries that share one staged copy of each union chunk: the caller's q_tile (default 128),
// halved until it divides the sequence (seq_len is a multiple of 64).
int effective_q_tile(const hils_prefill_params* p) {
  int qt = p->q_tile > 0 ? p->q_tile : 128;
  while (p->seq_len % qt != 0) qt >>= 1;
  return qt;
}

// (batch, head) pairs per chunk-major batch (one launch per stage per batch).  A batch is as
// large as two budgets allow, and at least one pair: its list and partial buffers within 8 GiB
// of workspace, and its q, k and v within 160 MiB, so that the chunks its work items stage
// stay in the 256 MB last-level cache (at 128K that is one pair per batch: two were 2 % and
// seven 12 % slower).  The batches are then evened out.
constexpr size_t kCmBatchBytes = (size_t)8 << 30;
constexpr size_t kCmCacheBytes = (size_t)160 << 20;
size_t cm_pair_bytes(const hils_prefill_params* p) {
  const size_t S = p->seq_len, k = p->topk, N = (S + p->chunk - 1) / p->chunk, d = p->head_dim;
  return (4 * N + 2) * 4 + S * k * 8 + hils::cm_max_items(S * k, N) * 8 + S * k * d * 2;
}
int cm_batch_pairs(const hils_prefill_params* p) {
  const size_t bh = (size_t)p->batch * p->heads;
  const size_t qkv = (size_t)p->seq_len * p->head_dim * 2 * 3;
  const size_t most = std::max<size_t>(1, std::min({bh, kCmBatchBytes / cm_pair_bytes(p), kCmCacheBytes / qkv}));
  const size_t batches = (bh + most - 1) / most;
  return (int)((bh + batches - 1) / batches);
}

PrefillLayout prefill_layout(const hils_prefill_params* p, bool with_sel) {
  PrefillLayout L{};
  const size_t B = p->batch, H = p->heads, S = p->seq_len, k = p->topk, r = p->qcal_rank;
  size_t off = 0;
  L.tcode = off;
  off += align_up(B * S * r * sizeof(float));
  L.idx = off;
  if (!with_sel) off += align_up(B * H * S * k * sizeof(int32_t));
  L.w = off;
  if (!with_sel) off += align_up(B * H * S * k * sizeof(float));
  if (p->attn_mode != HILS_ATTN_UNION) {       // chunk-major: a batch of (batch, head) pairs
    L.probe = off;                             // union probe counter (auto mode)
    off += align_up(4);
    const size_t N = (S + p->chunk - 1) / p->chunk, d = p->head_dim, P = cm_batch_pairs(p);
    L.cm_cnt = off;
    off += align_up(P * N * 4);
    L.cm_off = off;
    off += align_up(P * (N + 1) * 4);
    L.cm_cur = off;
    off += align_up(P * N * 4);
    L.cm_toff = off;
    off += align_up(P * (N + 1) * 4);
    L.cm_ent = off;
    off += align_up(P * S * k * 8);
    L.cm_desc = off;
    off += align_up(P * hils::cm_max_items(S * k, N) * 8);
    L.cm_partial = off;
    off += align_up(P * S * k * d * 2);
  }
  L.total = off;
  return L;
}

// A sequence that is not a multiple of the chunk is staged into copies padded to whole chunks
// (q, k, v, h in, o out; the selection stays in the workspace and its real rows are copied out
// when the caller asks for them).  The padded rows are zero and come after every real row, so no
// real row sees them; the last landmark (ceil(L / 64) of them) describes the partial chunk.
struct PadLayout {
  PrefillLayout inner;       // layout of the call on the padded sequence
  size_t qp, kp, vp, hp, op, total;
};

PadLayout pad_layout(const hils_prefill_params* p) {
  PadLayout P{};
  hils_prefill_params pp = *p;
  pp.seq_len = (p->seq_len + 63) / 64 * 64;
  P.inner = prefill_layout(&pp, false);
  const size_t B = p->batch, H = p->heads, Lp = pp.seq_len, d = p->head_dim, e = elem_bytes(p->dtype);
  const size_t Hk = p->kv_heads > 0 ? (size_t)p->kv_heads : H;
  size_t off = P.inner.total;
  P.qp = off;
  off += align_up(B * H * Lp * d * e);
  P.kp = off;
  off += align_up(B * Hk * Lp * d * e);
  P.vp = off;
  off += align_up(B * Hk * Lp * d * e);
  P.hp = off;
  off += align_up(p->qcal_rank > 0 ? B * Lp * p->hidden * e : 0);
  P.op = off;
  off += align_up(B * H * Lp * d * e);
  P.total = off;
  return P;
}

// Chunk sizes other than 64: the Q-Cal code, the selection (when not returned) and, for bf16,
// the chunk-major lists and partials.
PrefillLayout gchunk_layout(const hils_prefill_params* p, bool with_sel) {
  hils_prefill_params pp = *p;
  pp.attn_mode = p->dtype == HILS_DTYPE_BF16 ? HILS_ATTN_CHUNK_MAJOR : HILS_ATTN_UNION;
  return prefill_layout(&pp, with_sel);
}

// Chunk-major attention (bf16) over the selection in idx / w: the (batch, head) pairs in batches,
// one launch per stage and batch.
template <int D>
hipError_t run_chunk_major(const hils_prefill_params* p, const void* q, const void* k, const void* v, void* o,
                           const int32_t* idx, const float* w, char* ws, const PrefillLayout& L, float scale,
                           hipStream_t st) {
  hils::CmArgs ca;
  ca.q = q;
  ca.key = k;
  ca.val = v;
  ca.o = o;
  ca.idx = idx;
  ca.w = w;
  ca.cnt = reinterpret_cast<uint32_t*>(ws + L.cm_cnt);
  ca.off = reinterpret_cast<uint32_t*>(ws + L.cm_off);
  ca.cur = reinterpret_cast<uint32_t*>(ws + L.cm_cur);
  ca.toff = reinterpret_cast<uint32_t*>(ws + L.cm_toff);
  ca.ent = reinterpret_cast<uint32_t*>(ws + L.cm_ent);
  ca.desc = reinterpret_cast<uint32_t*>(ws + L.cm_desc);
  ca.partial = ws + L.cm_partial;
  ca.L = p->seq_len;
  ca.C = p->chunk;
  ca.N = (p->seq_len + p->chunk - 1) / p->chunk;
  ca.k = p->topk;
  ca.scale = scale;
  ca.H = p->heads;
  ca.G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  ca.bt = p->block_table;
  ca.bt_stride = p->block_table_stride;
  ca.num_pages = p->num_pages;
  const int BH = p->batch * p->heads, P = cm_batch_pairs(p);
  for (int pair0 = 0; pair0 < BH; pair0 += P) {
    ca.pair0 = pair0;
    ca.npairs = std::min(P, BH - pair0);
    const hipError_t e = hils::launch_chunk_attention_cm<D>(ca, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t prefill_workspace_bytes(const hils_prefill_params* p, bool with_sel) {
  if (p->chunk != 64) return gchunk_layout(p, with_sel).total;
  return p->seq_len % 64 == 0 ? prefill_layout(p, with_sel).total : pad_layout(p).total;
}

template <typename T>
hipError_t run_prefill_gchunk(const hils_prefill_params* p, const void* q, const void* k, const void* v,
                              const void* lmk, const void* h, const void* w_down, const void* w_up, void* o,
                              int32_t* idx, float* w, float* tcode, char* ws, const PrefillLayout& L,
                              hipStream_t st) {
  constexpr bool cm = sizeof(T) == 2;          // bf16: selection here, attention chunk-major
  hipError_t e;
  hipEvent_t* ev = p->n_stage_events >= 4 ? (hipEvent_t*)p->stage_events : nullptr;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  if (p->qcal_rank > 0) {
    e = hils::launch_prefill_qcal_code<T>(static_cast<const T*>(h), static_cast<const T*>(w_down), tcode,
                                          p->batch * p->seq_len, p->hidden, p->qcal_rank, st);
    if (e != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  hils::GcArgs a;
  a.q = q;
  a.key = k;
  a.val = v;
  a.lmk = lmk;
  a.w_up = w_up;
  a.tcode = tcode;
  a.o = cm ? nullptr : o;
  a.idx = idx;
  a.w = w;
  a.B = p->batch;
  a.H = p->heads;
  a.G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  a.L = p->seq_len;
  a.C = p->chunk;
  a.N = (p->seq_len + p->chunk - 1) / p->chunk;
  a.k = p->topk;
  a.r = p->qcal_rank;
  a.tstride = p->qcal_rank;
  a.force_local = p->force_local;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  if (cm && p->seq_len % 64 == 0) {
    // whole 64-query tiles: the MFMA selection (each tile scored against its last row's
    // candidates, later landmarks masked per query), amended for the forced local chunk
    hils::SelectArgs sa;
    sa.q = q;
    sa.lmk = lmk;
    sa.tcode = tcode;
    sa.w_up = w_up;
    sa.idx = idx;
    sa.w = w;
    sa.B = p->batch;
    sa.G = a.G;
    sa.H = p->heads;
    sa.L = p->seq_len;
    sa.N = a.N;
    sa.C = p->chunk;
    sa.k = p->topk;
    sa.r = p->qcal_rank;
    sa.scale = a.scale;
    e = p->head_dim == 64 ? hils::launch_select<T, 64>(sa, st) : hils::launch_select<T, 128>(sa, st);
    if (e == hipSuccess && p->force_local) {
      hils::LocalArgs la;
      la.q = q;
      la.lmk = lmk;
      la.w_up = w_up;
      la.tcode = tcode;
      la.kv_len = nullptr;
      la.idx = idx;
      la.w = w;
      la.B = p->batch;
      la.H = p->heads;
      la.L = p->seq_len;
      la.N = a.N;
      la.G = a.G;
      la.k = p->topk;
      la.r = p->qcal_rank;
      la.tstride = p->qcal_rank;
      la.lc = p->chunk == 32 ? 5 : 7;
      la.scale = a.scale;
      e = p->head_dim == 64 ? hils::launch_force_local<T, 64>(la, false, st)
                            : hils::launch_force_local<T, 128>(la, false, st);
    }
  } else {
    e = p->head_dim == 64 ? hils::launch_gchunk<T, 64>(a, st) : hils::launch_gchunk<T, 128>(a, st);
  }
  if (e != hipSuccess) return e;
  // fp32: selection and attention run in one kernel, so their two stage marks coincide
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  if constexpr (cm) {
    e = p->head_dim == 64 ? run_chunk_major<64>(p, q, k, v, o, idx, w, ws, L, a.scale, st)
                          : run_chunk_major<128>(p, q, k, v, o, idx, w, ws, L, a.scale, st);
    if (e != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
  return hipSuccess;
}

template <typename T, int D>
hipError_t run_prefill(const hils_prefill_params* p, const void* q, const void* k, const void* v,
                       const void* lmk, const void* h, const void* w_down, const void* w_up,
                       void* o, int32_t* idx, float* w, float* tcode, char* ws,
                       const PrefillLayout& L, hipStream_t st) {
  hipError_t e;
  hipEvent_t* ev = p->n_stage_events >= 4 ? (hipEvent_t*)p->stage_events : nullptr;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  const float scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)D);
  if (p->qcal_rank > 0) {
    e = hils::launch_prefill_qcal_code<T>(static_cast<const T*>(h), static_cast<const T*>(w_down),
                                          tcode, p->batch * p->seq_len, p->hidden, p->qcal_rank, st);
    if (e != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  hils::SelectArgs sa;
  sa.q = q;
  sa.lmk = lmk;
  sa.tcode = tcode;
  sa.w_up = w_up;
  sa.idx = idx;
  sa.w = w;
  sa.B = p->batch;
  sa.G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  sa.H = p->heads;
  sa.L = p->seq_len;
  sa.N = p->seq_len / 64;
  sa.C = 64;
  sa.k = p->topk;
  sa.r = p->qcal_rank;
  sa.scale = scale;
  if ((e = hils::launch_select<T, D>(sa, st)) != hipSuccess) return e;
  if (p->force_local) {
    hils::LocalArgs la;
    la.q = q;
    la.lmk = lmk;
    la.w_up = w_up;
    la.tcode = tcode;
    la.kv_len = nullptr;
    la.idx = idx;
    la.w = w;
    la.B = p->batch;
    la.H = p->heads;
    la.L = p->seq_len;
    la.N = p->seq_len / 64;
    la.G = sa.G;
    la.k = p->topk;
    la.r = p->qcal_rank;
    la.tstride = p->qcal_rank;
    la.lc = 6;
    la.scale = scale;
    if ((e = hils::launch_force_local<T, D>(la, false, st)) != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  hils::AttnArgs aa;
  aa.q = q;
  aa.key = k;
  aa.val = v;
  aa.idx = idx;
  aa.w = w;
  aa.o = o;
  aa.B = p->batch;
  aa.G = sa.G;
  aa.H = p->heads;
  aa.L = p->seq_len;
  aa.N = p->seq_len / 64;
  aa.topk = p->topk;
  aa.q_tile = effective_q_tile(p);
  aa.scale = scale;
  aa.block_table = p->block_table;
  aa.bt_stride = p->block_table_stride;
  aa.num_pages = p->num_pages;
  if constexpr (sizeof(T) == 2) {
    bool chunk_major = p->attn_mode == HILS_ATTN_CHUNK_MAJOR;
    if (p->attn_mode == HILS_ATTN_AUTO) {      // measure the selection's overlap, then choose
      // The choice waits on the host for one counter: not possible inside a stream capture
      // (checked before anything is enqueued, in hils_prefill_fwd).
      uint32_t* probe = reinterpret_cast<uint32_t*>(ws + L.probe);
      int groups = 0;
      if ((e = hils::launch_union_probe(idx, p->batch, p->heads, p->seq_len, p->topk, probe, &groups, st)) !=
          hipSuccess)
        return e;
      uint32_t total = 0;
      if ((e = hipMemcpyAsync(&total, probe, 4, hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
      if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
      chunk_major = groups > 0 && (double)total / groups > 8.0 * p->topk;
    }
    if (chunk_major) {
      if ((e = run_chunk_major<D>(p, q, k, v, o, idx, w, ws, L, scale, st)) != hipSuccess) return e;
      if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
      return hipSuccess;
    }
  }
  if ((e = hils::launch_chunk_attention<T, D>(aa, st)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------------------------
struct DecodeLayout {
  size_t tcode, scores, cand, idx, w, partial, total;
};

// Caches of up to this many chunks select from the scan's per-workgroup candidate lists; longer
// ones from dense scores.
constexpr int kDecodeCandMaxChunks = 8192;

int check_decode_params(const hils_decode_params* p) {
  if (!p) return fail(HILS_ERR_INVALID_ARG, "params is NULL");
  if (p->batch <= 0 || p->heads <= 0 || p->max_kv_len <= 0 || p->head_dim <= 0)
    return fail(HILS_ERR_INVALID_ARG, "batch, heads, max_kv_len and head_dim must be positive");
  if (p->dtype != HILS_DTYPE_BF16 && p->dtype != HILS_DTYPE_FP32)
    return fail(HILS_ERR_UNSUPPORTED, "dtype %d is not supported", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HILS_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", p->head_dim);
  if (p->chunk != 64 && p->chunk != 32 && p->chunk != 128)
    return fail(HILS_ERR_UNSUPPORTED, "chunk %d is not supported (32, 64 or 128)", p->chunk);
  if (p->chunk != 64) {
    if ((p->max_kv_len + p->chunk - 1) / p->chunk > 65535)
      return fail(HILS_ERR_UNSUPPORTED, "chunk %d: more than 65535 chunks per sequence", p->chunk);
  }
  if (p->topk < 1 || p->topk > 64)
    return fail(HILS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", p->topk);
  if ((p->max_kv_len + 63) / 64 > 65535)
    return fail(HILS_ERR_UNSUPPORTED, "more than 65535 chunks per sequence");
  if (p->qcal_rank < 0 || p->qcal_rank > 64)
    return fail(HILS_ERR_UNSUPPORTED, "qcal_rank %d outside [0, 64]", p->qcal_rank);
  if (p->qcal_rank > 0 && (p->hidden <= 0 || p->hidden % 128 != 0))
    return fail(HILS_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 128", p->hidden);
  if (!(isfinite(p->scale))) return fail(HILS_ERR_INVALID_ARG, "scale is not finite");
  if (p->n_stage_events < 0 || (p->n_stage_events > 0 && !p->stage_events))
    return fail(HILS_ERR_INVALID_ARG, "stage_events inconsistent with n_stage_events");
  if (p->kv_heads < 0 || p->kv_heads > p->heads || (p->kv_heads > 0 && p->heads % p->kv_heads != 0))
    return fail(HILS_ERR_INVALID_ARG, "kv_heads %d must divide heads %d", p->kv_heads, p->heads);
  if (p->force_local != 0 && p->force_local != 1)
    return fail(HILS_ERR_INVALID_ARG, "force_local must be 0 or 1");
  if (p->block_table && (p->num_pages < 1 || p->block_table_stride < (p->max_kv_len + p->chunk - 1) / p->chunk))
    return fail(HILS_ERR_INVALID_ARG, "paged cache: num_pages >= 1 and block_table_stride >= %d needed",
                (p->max_kv_len + p->chunk - 1) / p->chunk);
  if ((double)p->batch * p->heads > 2147483647.0)
    return fail(HILS_ERR_UNSUPPORTED, "problem too large");
  return HILS_OK;
}

DecodeLayout decode_layout(const hils_decode_params* p, bool with_sel) {
  DecodeLayout L{};
  const size_t B = p->batch, H = p->heads, d = p->head_dim, k = p->topk;
  const size_t N = (p->max_kv_len + p->chunk - 1) / p->chunk;
  size_t off = 0;
  L.tcode = off;
  off += align_up(B * (size_t)(p->qcal_rank > 0 ? hils::kTcodeStride : 0) * sizeof(float));
  const int qb = hils::decode_score_qb((int)(B * H), (int)N);
  const size_t stride = hils::decode_score_stride((int)N, qb);   // landmarks per pair, padded
  L.scores = L.cand = off;
  if (N <= (size_t)kDecodeCandMaxChunks) {
    L.cand = off;                              // 64 (key, chunk) entries per scan workgroup
    off += align_up(B * H * (stride / (qb * hils::kScoreBlock)) * 64 * 2 * sizeof(uint32_t));
  } else {
    L.scores = off;
    off += align_up(B * H * stride * sizeof(float));
  }
  L.idx = off;
  if (!with_sel) off += align_up(B * H * k * sizeof(int32_t));
  L.w = off;
  if (!with_sel) off += align_up(B * H * k * sizeof(float));
  L.partial = off;
  off += align_up(B * H * k * d * sizeof(float));
  L.total = off;
  return L;
}

// Chunk sizes 32 and 128: the scan and the selection of the 64-key path (chunk counts from
// kv_len and C), the forced local chunk's post-pass, then the split attention of
// launch_decode_attend_gc.
template <typename T, int D>
hipError_t run_decode_gc(const hils_decode_params* p, const void* q, const void* kc, const void* vc,
                         const void* lmk, const int32_t* kv_len, const void* h, const void* w_down,
                         const void* w_up, void* o, int32_t* idx, float* w, char* ws, const DecodeLayout& L,
                         hipStream_t st) {
  hipError_t e;
  hipEvent_t* ev = p->n_stage_events >= 5 ? (hipEvent_t*)p->stage_events : nullptr;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  float* tcode = reinterpret_cast<float*>(ws + L.tcode);
  e = hils::launch_decode_tcode<T>(static_cast<const T*>(h), static_cast<const T*>(w_down), tcode, p->batch,
                                   p->hidden, p->qcal_rank, st);
  if (e != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  hils::DecodeArgs a{};
  a.q = q;
  a.w_up = w_up;
  a.tcode = tcode;
  a.k_cache = kc;
  a.v_cache = vc;
  a.lmk = lmk;
  a.kv_len = kv_len;
  a.scores = reinterpret_cast<float*>(ws + L.scores);
  a.idx = idx;
  a.w = w;
  a.partial = reinterpret_cast<float*>(ws + L.partial);
  a.o = o;
  a.B = p->batch;
  a.G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  a.H = p->heads;
  a.Lmax = p->max_kv_len;
  a.C = p->chunk;
  a.Nmax = (p->max_kv_len + p->chunk - 1) / p->chunk;
  a.block_table = p->block_table;
  a.bt_stride = p->block_table_stride;
  a.num_pages = p->num_pages;
  a.k = p->topk;
  a.r = p->qcal_rank;
  a.score_qb = hils::decode_score_qb(a.B * a.H, a.Nmax);
  a.score_stride = hils::decode_score_stride(a.Nmax, a.score_qb);
  a.score_ymax = (int)(a.score_stride / (a.score_qb * hils::kScoreBlock));
  a.cand = a.Nmax <= kDecodeCandMaxChunks ? static_cast<void*>(ws + L.cand) : nullptr;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)D);
  a.force_local = p->force_local;
  if ((e = hils::launch_decode_scores<T, D>(a, st)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  if ((e = hils::launch_decode_select(a, st)) != hipSuccess) return e;
  if (p->force_local) {
    hils::LocalArgs la;
    la.q = q;
    la.lmk = lmk;
    la.w_up = w_up;
    la.tcode = tcode;
    la.kv_len = kv_len;
    la.idx = idx;
    la.w = w;
    la.B = p->batch;
    la.H = p->heads;
    la.L = p->max_kv_len;
    la.N = a.Nmax;
    la.G = a.G;
    la.k = p->topk;
    la.r = p->qcal_rank;
    la.tstride = hils::kTcodeStride;
    la.lc = p->chunk == 32 ? 5 : 7;
    la.scale = a.scale;
    if ((e = hils::launch_force_local<T, D>(la, true, st)) != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
  if ((e = hils::launch_decode_attend_gc<T, D>(a, p->chunk, st)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[4], st)) != hipSuccess) return e;
  return hipSuccess;
}

template <typename T, int D>
hipError_t run_decode(const hils_decode_params* p, const void* q, const void* kc, const void* vc,
                      const void* lmk, const int32_t* kv_len, const void* h, const void* w_down,
                      const void* w_up, void* o, int32_t* idx, float* w, char* ws,
                      const DecodeLayout& L, hipStream_t st) {
  hipError_t e;
  hipEvent_t* ev = p->n_stage_events >= 5 ? (hipEvent_t*)p->stage_events : nullptr;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  float* tcode = reinterpret_cast<float*>(ws + L.tcode);
  e = hils::launch_decode_tcode<T>(static_cast<const T*>(h), static_cast<const T*>(w_down), tcode,
                                   p->batch, p->hidden, p->qcal_rank, st);
  if (e != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  hils::DecodeArgs a;
  a.q = q;
  a.w_up = w_up;
  a.tcode = tcode;
  a.k_cache = kc;
  a.v_cache = vc;
  a.lmk = lmk;
  a.kv_len = kv_len;
  a.scores = reinterpret_cast<float*>(ws + L.scores);
  a.idx = idx;
  a.w = w;
  a.partial = reinterpret_cast<float*>(ws + L.partial);
  a.o = o;
  a.B = p->batch;
  a.G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  a.block_table = p->block_table;
  a.bt_stride = p->block_table_stride;
  a.num_pages = p->num_pages;
  a.H = p->heads;
  a.Lmax = p->max_kv_len;
  a.Nmax = (p->max_kv_len + 63) / 64;
  a.k = p->topk;
  a.r = p->qcal_rank;
  a.score_qb = hils::decode_score_qb(a.B * a.H, a.Nmax);
  a.score_stride = hils::decode_score_stride(a.Nmax, a.score_qb);
  a.score_ymax = (int)(a.score_stride / (a.score_qb * hils::kScoreBlock));
  const bool cand = a.Nmax <= kDecodeCandMaxChunks;
  a.cand = cand ? static_cast<void*>(ws + L.cand) : nullptr;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)D);
  a.force_local = p->force_local;
  a.C = 64;
  if (hils::decode_fused_ok<T>(a)) {           // scan, selection and attention in one kernel
    if ((e = hils::launch_decode_fused<T, D>(a, st)) != hipSuccess) return e;
    for (int s = 2; s <= 4; ++s)
      if (ev && (e = hipEventRecord(ev[s], st)) != hipSuccess) return e;
    return hipSuccess;
  }
  if ((e = hils::launch_decode_scores<T, D>(a, st)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  if (!hils::decode_select_fused<T>(a) && (e = hils::launch_decode_select(a, st)) != hipSuccess) return e;
  if (p->force_local) {
    hils::LocalArgs la;
    la.q = q;
    la.lmk = lmk;
    la.w_up = w_up;
    la.tcode = tcode;
    la.kv_len = kv_len;
    la.idx = idx;
    la.w = w;
    la.B = p->batch;
    la.H = p->heads;
    la.L = p->max_kv_len;
    la.N = a.Nmax;
    la.G = a.G;
    la.k = p->topk;
    la.r = p->qcal_rank;
    la.tstride = hils::kTcodeStride;
    la.lc = 6;
    la.scale = a.scale;
    if ((e = hils::launch_force_local<T, D>(la, true, st)) != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
  if ((e = hils::launch_decode_attend<T, D>(a, st)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[4], st)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace

extern "C" {

int hils_abi_version(void) { return HILS_ABI_VERSION; }

size_t hils_prefill_workspace_size(const hils_prefill_params* p, int with_selection) {
  g_last_error.clear();
  if (check_prefill_params(p) != HILS_OK) return 0;
  return prefill_workspace_bytes(p, with_selection != 0);
}

size_t hils_decode_workspace_size(const hils_decode_params* p, int with_selection) {
  g_last_error.clear();
  if (check_decode_params(p) != HILS_OK) return 0;
  return decode_layout(p, with_selection != 0).total;
}

int hils_prefill_fwd(const hils_prefill_params* p, const void* q, const void* k, const void* v,
                     const void* lmk, const void* h, const void* w_down, const void* w_up, void* o,
                     int32_t* sel_idx, float* sel_w, void* workspace, size_t workspace_bytes,
                     void* stream) {
  g_last_error.clear();
  int st = check_prefill_params(p);
  if (st != HILS_OK) return st;
  if (!q || !k || !v || !lmk || !o) return fail(HILS_ERR_INVALID_ARG, "a required tensor is NULL");
  const bool qcal = p->qcal_rank > 0;
  if (qcal != (h && w_down && w_up) || (!qcal && (h || w_down || w_up)))
    return fail(HILS_ERR_INVALID_ARG, "h, w_down and w_up must be given iff qcal_rank > 0");
  if ((sel_idx == nullptr) != (sel_w == nullptr))
    return fail(HILS_ERR_INVALID_ARG, "sel_idx and sel_w must be both NULL or both non-NULL");
  const bool with_sel = sel_idx != nullptr;
  const void* ptrs[] = {q, k, v, lmk, h, w_down, w_up, o, sel_idx, sel_w};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(HILS_ERR_ALIGNMENT, "a tensor is not 16-byte aligned");
  const size_t need = prefill_workspace_bytes(p, with_sel);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(HILS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (workspace && ((uintptr_t)workspace & (kWsAlign - 1)))
    return fail(HILS_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
  const size_t e = elem_bytes(p->dtype);
  const size_t B = p->batch, H = p->heads, S = p->seq_len, d = p->head_dim, kk = p->topk;
  const size_t r = p->qcal_rank, D = p->hidden;
  const size_t Hk = p->kv_heads > 0 ? (size_t)p->kv_heads : H;   // key/value heads
  const size_t kvb = p->block_table ? (size_t)p->num_pages * Hk * p->chunk * d * e : B * Hk * S * d * e;
  const Range in[] = {{q, B * H * S * d * e, "q"},   {k, kvb, "k"},
                      {v, kvb, "v"},  {lmk, B * Hk * ((S + p->chunk - 1) / p->chunk) * d * e, "lmk"},
                      {p->block_table, p->block_table ? B * (size_t)p->block_table_stride * 4 : 0, "block_table"},
                      {h, qcal ? B * S * D * e : 0, "h"}, {w_down, qcal ? r * D * e : 0, "w_down"},
                      {w_up, qcal ? H * d * r * e : 0, "w_up"}};
  const Range out[] = {{o, B * H * S * d * e, "o"},
                       {sel_idx, with_sel ? B * H * S * kk * 4 : 0, "sel_idx"},
                       {sel_w, with_sel ? B * H * S * kk * 4 : 0, "sel_w"},
                       {workspace, need, "workspace"}};
  for (const Range& a : out) {
    for (const Range& b : in)
      if (overlap(a, b)) return fail(HILS_ERR_INVALID_ARG, "%s overlaps input %s", a.name, b.name);
    for (const Range& b : out)
      if (&a != &b && overlap(a, b)) return fail(HILS_ERR_INVALID_ARG, "%s overlaps %s", a.name, b.name);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->attn_mode == HILS_ATTN_AUTO && p->chunk == 64) {   // (other chunk sizes take no mode)
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t ce = hipStreamIsCapturing(s, &cs);
    if (ce != hipSuccess) return hip_fail(ce, "hils_prefill_fwd: hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(HILS_ERR_UNSUPPORTED, "attn_mode HILS_ATTN_AUTO waits on the host and cannot be captured");
  }
  char* ws = static_cast<char*>(workspace);
  hipError_t err = hipSuccess;
  if (p->chunk != 64) {                        // any seq_len: partial last chunks need no padding
    const PrefillLayout G = gchunk_layout(p, with_sel);
    int32_t* gidx = with_sel ? sel_idx : reinterpret_cast<int32_t*>(ws + G.idx);
    float* gw = with_sel ? sel_w : reinterpret_cast<float*>(ws + G.w);
    float* gt = qcal ? reinterpret_cast<float*>(ws + G.tcode) : nullptr;
    err = p->dtype == HILS_DTYPE_BF16
              ? run_prefill_gchunk<hils::bf16>(p, q, k, v, lmk, h, w_down, w_up, o, gidx, gw, gt, ws, G, s)
              : run_prefill_gchunk<float>(p, q, k, v, lmk, h, w_down, w_up, o, gidx, gw, gt, ws, G, s);
    if (err != hipSuccess) return hip_fail(err, "hils_prefill_fwd");
    return HILS_OK;
  }
  const bool padded = p->seq_len % 64 != 0;
  hils_prefill_params pp = *p;
  PrefillLayout L;
  const void *qr = q, *kr = k, *vr = v, *hr = h;
  void* orun = o;
  int32_t* idx;
  float* w;
  if (padded) {
    const PadLayout P = pad_layout(p);
    pp.seq_len = (p->seq_len + 63) / 64 * 64;
    L = P.inner;
    const int Ls = p->seq_len, Lp = pp.seq_len;
    auto pad = [&](const void* src, size_t off, int nseq, size_t row_bytes) {
      if (err == hipSuccess) err = hils::launch_copy_rows(src, ws + off, nseq, Ls, Lp, row_bytes, s);
    };
    pad(q, P.qp, (int)(B * H), d * e);
    pad(k, P.kp, (int)(B * Hk), d * e);
    pad(v, P.vp, (int)(B * Hk), d * e);
    if (qcal) pad(h, P.hp, (int)B, D * e);
    if (err != hipSuccess) return hip_fail(err, "hils_prefill_fwd: padding");
    qr = ws + P.qp;
    kr = ws + P.kp;
    vr = ws + P.vp;
    hr = qcal ? ws + P.hp : nullptr;
    orun = ws + P.op;
    idx = reinterpret_cast<int32_t*>(ws + L.idx);
    w = reinterpret_cast<float*>(ws + L.w);
  } else {
    L = prefill_layout(p, with_sel);
    idx = with_sel ? sel_idx : reinterpret_cast<int32_t*>(ws + L.idx);
    w = with_sel ? sel_w : reinterpret_cast<float*>(ws + L.w);
  }
  float* tcode = qcal ? reinterpret_cast<float*>(ws + L.tcode) : nullptr;
  if (p->dtype == HILS_DTYPE_BF16) {
    err = p->head_dim == 64
              ? run_prefill<hils::bf16, 64>(&pp, qr, kr, vr, lmk, hr, w_down, w_up, orun, idx, w, tcode, ws, L, s)
              : run_prefill<hils::bf16, 128>(&pp, qr, kr, vr, lmk, hr, w_down, w_up, orun, idx, w, tcode, ws, L, s);
  } else {
    err = p->head_dim == 64
              ? run_prefill<float, 64>(&pp, qr, kr, vr, lmk, hr, w_down, w_up, orun, idx, w, tcode, ws, L, s)
              : run_prefill<float, 128>(&pp, qr, kr, vr, lmk, hr, w_down, w_up, orun, idx, w, tcode, ws, L, s);
  }
  if (err == hipSuccess && padded) {           // the real rows back to the caller
    err = hils::launch_copy_rows(orun, o, (int)(B * H), pp.seq_len, p->seq_len, d * e, s);
    if (err == hipSuccess && with_sel)
      err = hils::launch_copy_rows(idx, sel_idx, (int)(B * H), pp.seq_len, p->seq_len, kk * 4, s);
    if (err == hipSuccess && with_sel)
      err = hils::launch_copy_rows(w, sel_w, (int)(B * H), pp.seq_len, p->seq_len, kk * 4, s);
  }
  if (err != hipSuccess) return hip_fail(err, "hils_prefill_fwd");
  return HILS_OK;
}

}  // extern "C"

namespace {

int decode_entry(const hils_decode_params* p, const void* q, const void* k_cache, const void* v_cache,
                 const void* lmk, const int32_t* kv_len, const void* h, const void* w_down,
                 const void* w_up, void* o, int32_t* sel_idx, float* sel_w, void* workspace,
                 size_t workspace_bytes, void* stream, const char* who) {
  int st = check_decode_params(p);
  if (st != HILS_OK) return st;
  if (!q || !k_cache || !v_cache || !lmk || !kv_len || !o)
    return fail(HILS_ERR_INVALID_ARG, "a required tensor is NULL");
  const bool qcal = p->qcal_rank > 0;
  if (qcal != (h && w_down && w_up) || (!qcal && (h || w_down || w_up)))
    return fail(HILS_ERR_INVALID_ARG, "h, w_down and w_up must be given iff qcal_rank > 0");
  if ((sel_idx == nullptr) != (sel_w == nullptr))
    return fail(HILS_ERR_INVALID_ARG, "sel_idx and sel_w must be both NULL or both non-NULL");
  const bool with_sel = sel_idx != nullptr;
  const void* ptrs[] = {q, k_cache, v_cache, lmk, h, w_down, w_up, o, sel_idx, sel_w};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(HILS_ERR_ALIGNMENT, "a tensor is not 16-byte aligned");
  if ((uintptr_t)kv_len & 3u) return fail(HILS_ERR_ALIGNMENT, "kv_len is not 4-byte aligned");
  const DecodeLayout L = decode_layout(p, with_sel);
  if (!workspace || workspace_bytes < L.total)
    return fail(HILS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if ((uintptr_t)workspace & (kWsAlign - 1))
    return fail(HILS_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
  const size_t e = elem_bytes(p->dtype);
  const size_t B = p->batch, H = p->heads, Lm = p->max_kv_len, d = p->head_dim, kk = p->topk;
  const size_t N = (Lm + p->chunk - 1) / p->chunk, r = p->qcal_rank, D = p->hidden;
  const size_t Hk = p->kv_heads > 0 ? (size_t)p->kv_heads : H;   // key/value heads
  const size_t cache = p->block_table ? (size_t)p->num_pages * Hk * p->chunk * d * e : B * Hk * Lm * d * e;
  if (p->block_table && ((uintptr_t)p->block_table & 3))
    return fail(HILS_ERR_ALIGNMENT, "block_table is not 4-byte aligned");
  const Range in[] = {{q, B * H * d * e, "q"},           {k_cache, cache, "k_cache"},
                      {v_cache, cache, "v_cache"},       {lmk, B * Hk * N * d * e, "lmk"},
                      {p->block_table, p->block_table ? B * (size_t)p->block_table_stride * 4 : 0, "block_table"},
                      {kv_len, B * 4, "kv_len"},          {h, qcal ? B * D * e : 0, "h"},
                      {w_down, qcal ? r * D * e : 0, "w_down"}, {w_up, qcal ? H * d * r * e : 0, "w_up"}};
  const Range out[] = {{o, B * H * d * e, "o"},
                       {sel_idx, with_sel ? B * H * kk * 4 : 0, "sel_idx"},
                       {sel_w, with_sel ? B * H * kk * 4 : 0, "sel_w"},
                       {workspace, L.total, "workspace"}};
  for (const Range& a : out) {
    for (const Range& b : in)
      if (overlap(a, b)) return fail(HILS_ERR_INVALID_ARG, "%s overlaps input %s", a.name, b.name);
    for (const Range& b : out)
      if (&a != &b && overlap(a, b)) return fail(HILS_ERR_INVALID_ARG, "%s overlaps %s", a.name, b.name);
  }
  char* ws = static_cast<char*>(workspace);
  int32_t* idx = with_sel ? sel_idx : reinterpret_cast<int32_t*>(ws + L.idx);
  float* w = with_sel ? sel_w : reinterpret_cast<float*>(ws + L.w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (p->chunk != 64) {
    if (p->dtype == HILS_DTYPE_BF16)
      err = p->head_dim == 64
                ? run_decode_gc<hils::bf16, 64>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s)
                : run_decode_gc<hils::bf16, 128>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s);
    else
      err = p->head_dim == 64
                ? run_decode_gc<float, 64>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s)
                : run_decode_gc<float, 128>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s);
  } else if (p->dtype == HILS_DTYPE_BF16) {
    err = p->head_dim == 64
              ? run_decode<hils::bf16, 64>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s)
              : run_decode<hils::bf16, 128>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s);
  } else {
    err = p->head_dim == 64
              ? run_decode<float, 64>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s)
              : run_decode<float, 128>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s);
  }
  if (err != hipSuccess) return hip_fail(err, who);
  return HILS_OK;
}

// Scratch of hils_decode_fwd_noalloc: one copy per GPU, held until the process ends.  In host
// code `scratch` only names the symbol; its device address on each GPU comes from
// hipGetSymbolAddress with that GPU current, once, and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)HILS_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hils_decode_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HILS_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hils_decode_fwd_noalloc: hipGetSymbolAddress(scratch)");
    if (!ptr || ((uintptr_t)ptr & (kWsAlign - 1)))
      return fail(HILS_ERR_HIP, "hils_decode_fwd_noalloc: static scratch at %p is not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HILS_OK;
}

}  // namespace

extern "C" {

int hils_decode_fwd(const hils_decode_params* p, const void* q, const void* k_cache,
                    const void* v_cache, const void* lmk, const int32_t* kv_len, const void* h,
                    const void* w_down, const void* w_up, void* o, int32_t* sel_idx, float* sel_w,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return decode_entry(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, sel_idx, sel_w, workspace,
                      workspace_bytes, stream, "hils_decode_fwd");
}

int hils_decode_fwd_noalloc(const hils_decode_params* p, const void* q, const void* k_cache,
                            const void* v_cache, const void* lmk, const int32_t* kv_len, const void* h,
                            const void* w_down, const void* w_up, void* o, int32_t* sel_idx, float* sel_w,
                            void* stream) {
  g_last_error.clear();
  int st = check_decode_params(p);
  if (st != HILS_OK) return st;
  if ((sel_idx == nullptr) != (sel_w == nullptr))
    return fail(HILS_ERR_INVALID_ARG, "sel_idx and sel_w must be both NULL or both non-NULL");
  const size_t need = decode_layout(p, sel_idx != nullptr).total;
  if (need > kStaticScratchBytes)
    return fail(HILS_ERR_WORKSPACE, "hils_decode_fwd_noalloc: %zu bytes of scratch needed, the static scratch holds %zu",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != HILS_OK) return st;
  return decode_entry(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, sel_idx, sel_w, ws,
                      kStaticScratchBytes, stream, "hils_decode_fwd_noalloc");
}

}  // extern "C"

namespace {

int check_dense_params(const hils_dense_params* p, bool prefill) {
  if (!p) return fail(HILS_ERR_INVALID_ARG, "params is NULL");
  if (p->batch <= 0 || p->heads <= 0 || p->seq_len <= 0 || p->head_dim <= 0)
    return fail(HILS_ERR_INVALID_ARG, "batch, heads, seq_len and head_dim must be positive");
  if (p->dtype != HILS_DTYPE_BF16 && p->dtype != HILS_DTYPE_FP32)
    return fail(HILS_ERR_UNSUPPORTED, "dtype %d is not supported", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HILS_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", p->head_dim);
  if (prefill && p->seq_len % 64 != 0)
    return fail(HILS_ERR_UNSUPPORTED, "seq_len %d is not a multiple of 64", p->seq_len);
  if (p->kv_heads < 0 || p->kv_heads > p->heads || (p->kv_heads > 0 && p->heads % p->kv_heads != 0))
    return fail(HILS_ERR_INVALID_ARG, "kv_heads %d must divide heads %d", p->kv_heads, p->heads);
  if (!(isfinite(p->scale))) return fail(HILS_ERR_INVALID_ARG, "scale is not finite");
  if ((double)p->batch * p->heads * (double)p->seq_len > 4e18 / 1024 ||
      (double)p->batch * p->heads * (p->seq_len / 64 + 1) > 2147483647.0)
    return fail(HILS_ERR_UNSUPPORTED, "problem too large");
  return HILS_OK;
}

size_t dense_decode_ws(const hils_dense_params* p) {
  const int pairs = p->batch * p->heads;
  return align_up((size_t)pairs * hils::dense_decode_splits(pairs, p->seq_len) * (p->head_dim + 2) * 4);
}

int check_overlaps(const Range* in, size_t nin, const Range* out, size_t nout) {
  for (size_t a = 0; a < nout; ++a) {
    for (size_t b = 0; b < nin; ++b)
      if (overlap(out[a], in[b])) return fail(HILS_ERR_INVALID_ARG, "%s overlaps input %s", out[a].name, in[b].name);
    for (size_t b = 0; b < nout; ++b)
      if (a != b && overlap(out[a], out[b]))
        return fail(HILS_ERR_INVALID_ARG, "%s overlaps %s", out[a].name, out[b].name);
  }
  return HILS_OK;
}

}  // namespace

extern "C" {

int hils_dense_prefill_fwd(const hils_dense_params* p, const void* q, const void* k, const void* v, void* o,
                           void* stream) {
  g_last_error.clear();
  int st = check_dense_params(p, true);
  if (st != HILS_OK) return st;
  if (!q || !k || !v || !o) return fail(HILS_ERR_INVALID_ARG, "a required tensor is NULL");
  for (const void* ptr : {q, k, v, (const void*)o})
    if (!aligned16(ptr)) return fail(HILS_ERR_ALIGNMENT, "a tensor is not 16-byte aligned");
  const size_t e = elem_bytes(p->dtype), B = p->batch, H = p->heads, S = p->seq_len, d = p->head_dim;
  const size_t Hk = p->kv_heads > 0 ? (size_t)p->kv_heads : H;
  const Range in[] = {{q, B * H * S * d * e, "q"}, {k, B * Hk * S * d * e, "k"}, {v, B * Hk * S * d * e, "v"}};
  const Range out[] = {{o, B * H * S * d * e, "o"}};
  if ((st = check_overlaps(in, 3, out, 1)) != HILS_OK) return st;
  hils::DenseArgs a;
  a.q = q;
  a.key = k;
  a.val = v;
  a.o = o;
  a.B = p->batch;
  a.H = p->heads;
  a.L = p->seq_len;
  a.G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (p->dtype == HILS_DTYPE_BF16)
    err = d == 64 ? hils::launch_dense_prefill<hils::bf16, 64>(a, s) : hils::launch_dense_prefill<hils::bf16, 128>(a, s);
  else
    err = d == 64 ? hils::launch_dense_prefill<float, 64>(a, s) : hils::launch_dense_prefill<float, 128>(a, s);
  if (err != hipSuccess) return hip_fail(err, "hils_dense_prefill_fwd");
  return HILS_OK;
}

int hils_hope_rotate(const hils_hope_params* p, void* x, const int32_t* positions, void* stream) {
  g_last_error.clear();
  if (!p) return fail(HILS_ERR_INVALID_ARG, "params is NULL");
  if (!x) return fail(HILS_ERR_INVALID_ARG, "x is NULL");
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1)
    return fail(HILS_ERR_INVALID_ARG, "batch, heads and seq_len must be positive");
  if (p->dtype != HILS_DTYPE_BF16 && p->dtype != HILS_DTYPE_FP32)
    return fail(HILS_ERR_UNSUPPORTED, "dtype %d is not bf16 or fp32", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HILS_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", p->head_dim);
  if (!(p->rope_base > 1.f)) return fail(HILS_ERR_INVALID_ARG, "rope_base must be above 1");
  if (p->train_len < 1) return fail(HILS_ERR_INVALID_ARG, "train_len must be positive");
  if (!aligned16(x)) return fail(HILS_ERR_ALIGNMENT, "x is not 16-byte aligned");
  hils::HopeArgs a;
  a.x = x;
  a.positions = positions;
  a.B = p->batch;
  a.H = p->heads;
  a.L = p->seq_len;
  a.pos0 = p->pos0;
  a.rotated = 0ull;
  const int d = p->head_dim;
  for (int i = 0; i < 64; ++i) {
    a.theta[i] = i < d / 2 ? pow((double)p->rope_base, -2.0 * i / d) : 0.0;
    if (i < d / 2 && 6.283185307179586476925286766559 / a.theta[i] <= (double)p->train_len) a.rotated |= 1ull << i;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (p->dtype == HILS_DTYPE_BF16)
    err = d == 64 ? hils::launch_hope_rotate<hils::bf16, 64>(a, s) : hils::launch_hope_rotate<hils::bf16, 128>(a, s);
  else
    err = d == 64 ? hils::launch_hope_rotate<float, 64>(a, s) : hils::launch_hope_rotate<float, 128>(a, s);
  if (err != hipSuccess) return hip_fail(err, "hils_hope_rotate");
  return HILS_OK;
}

int hils_partial_landmark(const hils_landmark_params* p, const void* k_cache, void* lmk, const int32_t* kv_len,
                          void* stream) {
  g_last_error.clear();
  if (!p) return fail(HILS_ERR_INVALID_ARG, "params is NULL");
  if (!k_cache || !lmk || !kv_len) return fail(HILS_ERR_INVALID_ARG, "a required tensor is NULL");
  if (p->batch < 1 || p->kv_heads < 1 || p->max_kv_len < 1)
    return fail(HILS_ERR_INVALID_ARG, "batch, kv_heads and max_kv_len must be positive");
  if (p->dtype != HILS_DTYPE_BF16 && p->dtype != HILS_DTYPE_FP32)
    return fail(HILS_ERR_UNSUPPORTED, "dtype %d is not bf16 or fp32", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HILS_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", p->head_dim);
  if (p->chunk != 32 && p->chunk != 64 && p->chunk != 128)
    return fail(HILS_ERR_UNSUPPORTED, "chunk %d is not supported (32, 64 or 128)", p->chunk);
  if ((double)p->batch * p->kv_heads * p->max_kv_len * p->head_dim > 4e18 / 8 ||
      (double)p->batch * p->kv_heads > 2147483647.0)
    return fail(HILS_ERR_UNSUPPORTED, "problem too large");
  if (!aligned16(k_cache) || !aligned16(lmk)) return fail(HILS_ERR_ALIGNMENT, "a tensor is not 16-byte aligned");
  if ((uintptr_t)kv_len & 3u) return fail(HILS_ERR_ALIGNMENT, "kv_len is not 4-byte aligned");
  const size_t e = elem_bytes(p->dtype), B = p->batch, Hk = p->kv_heads, d = p->head_dim;
  const size_t N = ((size_t)p->max_kv_len + p->chunk - 1) / p->chunk;
  const Range kr{k_cache, B * Hk * (size_t)p->max_kv_len * d * e, "k_cache"}, lr{lmk, B * Hk * N * d * e, "lmk"},
      vr{kv_len, B * 4, "kv_len"};
  if (overlap(lr, kr) || overlap(lr, vr)) return fail(HILS_ERR_INVALID_ARG, "lmk overlaps an input");
  hils::PartialLmkArgs a;
  a.k_cache = k_cache;
  a.lmk = lmk;
  a.kv_len = kv_len;
  a.B = p->batch;
  a.Hk = p->kv_heads;
  a.Lmax = p->max_kv_len;
  a.N = (int)N;
  a.C = p->chunk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (p->dtype == HILS_DTYPE_BF16)
    err = d == 64 ? hils::launch_partial_landmark<hils::bf16, 64>(a, s)
                  : hils::launch_partial_landmark<hils::bf16, 128>(a, s);
  else
    err = d == 64 ? hils::launch_partial_landmark<float, 64>(a, s) : hils::launch_partial_landmark<float, 128>(a, s);
  if (err != hipSuccess) return hip_fail(err, "hils_partial_landmark");
  return HILS_OK;
}

size_t hils_dense_decode_workspace_size(const hils_dense_params* p) {
  g_last_error.clear();
  if (check_dense_params(p, false) != HILS_OK) return 0;
  return dense_decode_ws(p);
}

int hils_dense_decode_fwd(const hils_dense_params* p, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* kv_len, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = check_dense_params(p, false);
  if (st != HILS_OK) return st;
  if (!q || !k_cache || !v_cache || !kv_len || !o) return fail(HILS_ERR_INVALID_ARG, "a required tensor is NULL");
  for (const void* ptr : {q, k_cache, v_cache, (const void*)o})
    if (!aligned16(ptr)) return fail(HILS_ERR_ALIGNMENT, "a tensor is not 16-byte aligned");
  if ((uintptr_t)kv_len & 3u) return fail(HILS_ERR_ALIGNMENT, "kv_len is not 4-byte aligned");
  const size_t need = dense_decode_ws(p);
  if (!workspace || workspace_bytes < need)
    return fail(HILS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if ((uintptr_t)workspace & (kWsAlign - 1)) return fail(HILS_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
  const size_t e = elem_bytes(p->dtype), B = p->batch, H = p->heads, S = p->seq_len, d = p->head_dim;
  const size_t Hk = p->kv_heads > 0 ? (size_t)p->kv_heads : H;
  const Range in[] = {{q, B * H * d * e, "q"}, {k_cache, B * Hk * S * d * e, "k_cache"},
                      {v_cache, B * Hk * S * d * e, "v_cache"}, {kv_len, B * 4, "kv_len"}};
  const Range out[] = {{o, B * H * d * e, "o"}, {workspace, need, "workspace"}};
  if ((st = check_overlaps(in, 4, out, 2)) != HILS_OK) return st;
  hils::DenseDecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_len = kv_len;
  a.partial = static_cast<float*>(workspace);
  a.o = o;
  a.B = p->batch;
  a.H = p->heads;
  a.Lmax = p->seq_len;
  a.G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (p->dtype == HILS_DTYPE_BF16)
    err = d == 64 ? hils::launch_dense_decode<hils::bf16, 64>(a, s) : hils::launch_dense_decode<hils::bf16, 128>(a, s);
  else
    err = d == 64 ? hils::launch_dense_decode<float, 64>(a, s) : hils::launch_dense_decode<float, 128>(a, s);
  if (err != hipSuccess) return hip_fail(err, "hils_dense_decode_fwd");
  return HILS_OK;
}

}  // extern "C"

namespace {

struct BwdLayout {
  size_t tcode, qt, dqbuf, lse, dw, dsig, dt, rbcnt, choff, ent, gpart, total;
};

BwdLayout bwd_layout(const hils_prefill_params* p) {
  BwdLayout L{};
  const size_t B = p->batch, H = p->heads, S = p->seq_len, d = p->head_dim, k = p->topk, r = p->qcal_rank;
  const size_t e = elem_bytes(p->dtype), N = S / 64;
  const int G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.tcode = take(r ? B * S * r * 4 : 0);
  L.qt = take(r ? B * H * S * d * e : 0);
  L.dqbuf = take(B * H * S * d * 4);
  L.lse = take(B * H * S * k * 4);
  L.dw = take(B * H * S * k * 4);
  L.dsig = take(B * H * S * k * 4);
  L.dt = take(r ? B * S * r * 4 : 0);
  const size_t nkv = B * (H / G);             // every key/value head's lists at once
  L.rbcnt = take(nkv * hils::bwd_rbcnt_words(G, (int)S, (int)N) * 4);
  L.choff = take(nkv * (N + 1) * 4);
  L.ent = take(nkv * (size_t)G * S * k * 4);
  const size_t X = std::max(H * d, (size_t)(r ? p->hidden : 0));
  L.gpart = take(r ? (size_t)hils::bwd_splits((int)(B * S)) * X * 64 * 4 : 0);
  L.total = off;
  return L;
}

int check_bwd_params(const hils_prefill_params* p) {
  int st = check_prefill_params(p);
  if (st != HILS_OK) return st;
  if (p->chunk != 64) return fail(HILS_ERR_UNSUPPORTED, "the backward pass needs chunk 64");
  if (p->seq_len % 64 != 0)
    return fail(HILS_ERR_UNSUPPORTED, "the backward pass needs seq_len a multiple of the chunk (64)");
  if (p->block_table) return fail(HILS_ERR_UNSUPPORTED, "the backward pass takes contiguous keys and values");
  if (p->seq_len / 64 > 16384) return fail(HILS_ERR_UNSUPPORTED, "the backward pass supports at most 16384 chunks");
  return HILS_OK;
}

}  // namespace

extern "C" {

size_t hils_prefill_bwd_workspace_size(const hils_prefill_params* p) {
  g_last_error.clear();
  if (check_bwd_params(p) != HILS_OK) return 0;
  return bwd_layout(p).total;
}

int hils_prefill_bwd(const hils_prefill_params* p, const void* q, const void* k, const void* v, const void* lmk,
                     const void* h, const void* w_down, const void* w_up, const int32_t* sel_idx,
                     const float* sel_w, const void* dout, void* dq, void* dk, void* dv, void* dlmk, void* dh,
                     void* dw_down, void* dw_up, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = check_bwd_params(p);
  if (st != HILS_OK) return st;
  if (!q || !k || !v || !lmk || !sel_idx || !sel_w || !dout || !dq || !dk || !dv || !dlmk)
    return fail(HILS_ERR_INVALID_ARG, "a required tensor is NULL");
  const bool qcal = p->qcal_rank > 0;
  const bool all_q = h && w_down && w_up && dh && dw_down && dw_up;
  const bool none_q = !h && !w_down && !w_up && !dh && !dw_down && !dw_up;
  if (qcal ? !all_q : !none_q)
    return fail(HILS_ERR_INVALID_ARG, "h, w_down, w_up, dh, dw_down and dw_up must be given iff qcal_rank > 0");
  const void* ptrs[] = {q, k, v, lmk, h, w_down, w_up, sel_idx, sel_w, dout, dq, dk, dv, dlmk, dh, dw_down, dw_up};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(HILS_ERR_ALIGNMENT, "a tensor is not 16-byte aligned");
  const BwdLayout L = bwd_layout(p);
  if (!workspace || workspace_bytes < L.total)
    return fail(HILS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if ((uintptr_t)workspace & (kWsAlign - 1)) return fail(HILS_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
  const size_t e = elem_bytes(p->dtype);
  const size_t B = p->batch, H = p->heads, S = p->seq_len, d = p->head_dim, kk = p->topk;
  const size_t r = p->qcal_rank, D = p->hidden;
  const size_t Hk = p->kv_heads > 0 ? (size_t)p->kv_heads : H;
  const size_t qb = B * H * S * d * e, kb = B * Hk * S * d * e, lb = B * Hk * (S / 64) * d * e;
  const Range in[] = {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {lmk, lb, "lmk"},
                      {h, qcal ? B * S * D * e : 0, "h"}, {w_down, qcal ? r * D * e : 0, "w_down"},
                      {w_up, qcal ? H * d * r * e : 0, "w_up"}, {sel_idx, B * H * S * kk * 4, "sel_idx"},
                      {sel_w, B * H * S * kk * 4, "sel_w"}, {dout, qb, "dout"}};
  const Range out[] = {{dq, qb, "dq"}, {dk, kb, "dk"}, {dv, kb, "dv"}, {dlmk, lb, "dlmk"},
                       {dh, qcal ? B * S * D * e : 0, "dh"}, {dw_down, qcal ? r * D * e : 0, "dw_down"},
                       {dw_up, qcal ? H * d * r * e : 0, "dw_up"}, {workspace, L.total, "workspace"}};
  if ((st = check_overlaps(in, sizeof(in) / sizeof(in[0]), out, sizeof(out) / sizeof(out[0]))) != HILS_OK) return st;
  char* ws = static_cast<char*>(workspace);
  hils::BwdArgs a;
  a.q = q;
  a.k_in = k;
  a.v_in = v;
  a.lmk = lmk;
  a.h = h;
  a.w_down = w_down;
  a.w_up = w_up;
  a.idx = sel_idx;
  a.w = sel_w;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlmk = dlmk;
  a.dh = dh;
  a.dw_down = dw_down;
  a.dw_up = dw_up;
  a.tcode = reinterpret_cast<float*>(ws + L.tcode);
  a.qt = ws + L.qt;
  a.dqbuf = reinterpret_cast<float*>(ws + L.dqbuf);
  a.lse = reinterpret_cast<float*>(ws + L.lse);
  a.dw = reinterpret_cast<float*>(ws + L.dw);
  a.dsig = reinterpret_cast<float*>(ws + L.dsig);
  a.dt = reinterpret_cast<float*>(ws + L.dt);
  a.rbcnt = reinterpret_cast<uint32_t*>(ws + L.rbcnt);
  a.choff = reinterpret_cast<uint32_t*>(ws + L.choff);
  a.ent = reinterpret_cast<uint32_t*>(ws + L.ent);
  a.gpart = reinterpret_cast<float*>(ws + L.gpart);
  a.B = p->batch;
  a.H = p->heads;
  a.L = p->seq_len;
  a.G = p->kv_heads > 0 ? p->heads / p->kv_heads : 1;
  a.d = p->head_dim;
  a.k = p->topk;
  a.r = p->qcal_rank;
  a.Dh = p->hidden;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (qcal) {
    if (p->dtype == HILS_DTYPE_BF16)
      err = hils::launch_prefill_qcal_code<hils::bf16>(static_cast<const hils::bf16*>(h),
                                                       static_cast<const hils::bf16*>(w_down), a.tcode,
                                                       p->batch * p->seq_len, p->hidden, p->qcal_rank, s);
    else
      err = hils::launch_prefill_qcal_code<float>(static_cast<const float*>(h), static_cast<const float*>(w_down),
                                                  a.tcode, p->batch * p->seq_len, p->hidden, p->qcal_rank, s);
  }
  if (err == hipSuccess) {
    if (p->dtype == HILS_DTYPE_BF16)
      err = d == 64 ? hils::launch_prefill_bwd<hils::bf16, 64>(a, s) : hils::launch_prefill_bwd<hils::bf16, 128>(a, s);
    else
      err = d == 64 ? hils::launch_prefill_bwd<float, 64>(a, s) : hils::launch_prefill_bwd<float, 128>(a, s);
  }
  if (err != hipSuccess) return hip_fail(err, "hils_prefill_bwd");
  return HILS_OK;
}

const char* hils_status_string(int status) {
  switch (status) {
    case HILS_OK: return "ok";
    case HILS_ERR_INVALID_ARG: return "invalid argument";
    case HILS_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case HILS_ERR_ALIGNMENT: return "misaligned pointer";
    case HILS_ERR_WORKSPACE: return "workspace missing or too small";
    case HILS_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* hils_last_hip_error(void) { return g_last_error.c_str(); }

}  // extern "C"
