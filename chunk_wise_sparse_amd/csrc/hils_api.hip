// C ABI of the HiLS forward pass: argument validation, workspace layout and launch sequencing.
// Every host-checkable error is reported before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "hils.h"
#include "hils_launch.h"

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
  size_t tcode, idx, w, probe, cm_cnt, cm_off, cm_cur, cm_toff, cm_ent, cm_partial, total;
};

int check_prefill_params(const hils_prefill_params* p) {
  if (!p) return fail(HILS_ERR_INVALID_ARG, "params is NULL");
  if (p->batch <= 0 || p->heads <= 0 || p->seq_len <= 0 || p->head_dim <= 0)
    return fail(HILS_ERR_INVALID_ARG, "batch, heads, seq_len and head_dim must be positive");
  if (p->dtype != HILS_DTYPE_BF16 && p->dtype != HILS_DTYPE_FP32)
    return fail(HILS_ERR_UNSUPPORTED, "dtype %d is not supported", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HILS_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", p->head_dim);
  if (p->chunk != 64) return fail(HILS_ERR_UNSUPPORTED, "chunk %d is not supported (64)", p->chunk);
  if (p->topk < 1 || p->topk > 64)
    return fail(HILS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", p->topk);
  if (p->seq_len % p->chunk != 0)
    return fail(HILS_ERR_UNSUPPORTED, "seq_len %d is not a multiple of the chunk size", p->seq_len);
  if (p->seq_len / p->chunk > 65535)
    return fail(HILS_ERR_UNSUPPORTED, "more than 65535 chunks per sequence");
  if (p->dtype == HILS_DTYPE_FP32 && p->head_dim == 128 && p->seq_len / p->chunk > 16384)
    return fail(HILS_ERR_UNSUPPORTED, "fp32 with head_dim 128 supports at most 16384 chunks");
  if (p->q_tile != 0 && p->q_tile != 64)
    return fail(HILS_ERR_UNSUPPORTED, "q_tile %d is not supported (64)", p->q_tile);
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
  const double bhld = (double)p->batch * p->heads * p->seq_len * p->head_dim;
  if (bhld > 4e18 / 8 || (double)p->batch * p->heads * (p->seq_len / 64) > 2147483647.0)
    return fail(HILS_ERR_UNSUPPORTED, "problem too large");
  return HILS_OK;
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
  if (p->attn_mode != HILS_ATTN_UNION) {       // chunk-major: one (batch, head) pair at a time
    L.probe = off;                             // union probe counter (auto mode)
    off += align_up(4);
    const size_t N = S / 64, d = p->head_dim;
    L.cm_cnt = off;
    off += align_up(N * 4);
    L.cm_off = off;
    off += align_up((N + 1) * 4);
    L.cm_cur = off;
    off += align_up(N * 4);
    L.cm_toff = off;
    off += align_up((N + 1) * 4);
    L.cm_ent = off;
    off += align_up(S * k * 4);
    L.cm_partial = off;
    off += align_up(S * k * d * 2);
  }
  L.total = off;
  return L;
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
  sa.k = p->topk;
  sa.r = p->qcal_rank;
  sa.scale = scale;
  if ((e = hils::launch_select<T, D>(sa, st)) != hipSuccess) return e;
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
  aa.scale = scale;
  if constexpr (sizeof(T) == 2) {
    bool chunk_major = p->attn_mode == HILS_ATTN_CHUNK_MAJOR;
    if (p->attn_mode == HILS_ATTN_AUTO) {      // measure the selection's overlap, then choose
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
      hils::CmArgs ca;
      ca.cnt = reinterpret_cast<uint32_t*>(ws + L.cm_cnt);
      ca.off = reinterpret_cast<uint32_t*>(ws + L.cm_off);
      ca.cur = reinterpret_cast<uint32_t*>(ws + L.cm_cur);
      ca.toff = reinterpret_cast<uint32_t*>(ws + L.cm_toff);
      ca.ent = reinterpret_cast<uint32_t*>(ws + L.cm_ent);
      ca.partial = ws + L.cm_partial;
      ca.L = p->seq_len;
      ca.N = p->seq_len / 64;
      ca.k = p->topk;
      ca.scale = scale;
      const size_t ld = (size_t)p->seq_len * D, lk = (size_t)p->seq_len * p->topk;
      for (size_t bh = 0; bh < (size_t)p->batch * p->heads; ++bh) {
        ca.q = static_cast<const T*>(q) + bh * ld;
        const size_t kvbh = (bh / p->heads) * (p->heads / aa.G) + (bh % p->heads) / aa.G;
        ca.key = static_cast<const T*>(k) + kvbh * ld;
        ca.val = static_cast<const T*>(v) + kvbh * ld;
        ca.o = static_cast<T*>(o) + bh * ld;
        ca.idx = idx + bh * lk;
        ca.w = w + bh * lk;
        if ((e = hils::launch_chunk_attention_cm<D>(ca, st)) != hipSuccess) return e;
      }
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
  if (p->chunk != 64) return fail(HILS_ERR_UNSUPPORTED, "chunk %d is not supported (64)", p->chunk);
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
  if (p->block_table && (p->num_pages < 1 || p->block_table_stride < (p->max_kv_len + 63) / 64))
    return fail(HILS_ERR_INVALID_ARG, "paged cache: num_pages >= 1 and block_table_stride >= %d needed",
                (p->max_kv_len + 63) / 64);
  if ((double)p->batch * p->heads > 2147483647.0)
    return fail(HILS_ERR_UNSUPPORTED, "problem too large");
  return HILS_OK;
}

DecodeLayout decode_layout(const hils_decode_params* p, bool with_sel) {
  DecodeLayout L{};
  const size_t B = p->batch, H = p->heads, d = p->head_dim, k = p->topk;
  const size_t N = (p->max_kv_len + 63) / 64;
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
  if (hils::decode_fused_ok<T>(a)) {           // scan, selection and attention in one kernel
    if ((e = hils::launch_decode_fused<T, D>(a, st)) != hipSuccess) return e;
    for (int s = 2; s <= 4; ++s)
      if (ev && (e = hipEventRecord(ev[s], st)) != hipSuccess) return e;
    return hipSuccess;
  }
  if ((e = hils::launch_decode_scores<T, D>(a, st)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  if (!hils::decode_select_fused<T>(a) && (e = hils::launch_decode_select(a, st)) != hipSuccess) return e;
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
  return prefill_layout(p, with_selection != 0).total;
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
  const PrefillLayout L = prefill_layout(p, with_sel);
  if (L.total > 0 && (!workspace || workspace_bytes < L.total))
    return fail(HILS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (workspace && ((uintptr_t)workspace & (kWsAlign - 1)))
    return fail(HILS_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
  const size_t e = elem_bytes(p->dtype);
  const size_t B = p->batch, H = p->heads, S = p->seq_len, d = p->head_dim, kk = p->topk;
  const size_t r = p->qcal_rank, D = p->hidden;
  const size_t Hk = p->kv_heads > 0 ? (size_t)p->kv_heads : H;   // key/value heads
  const Range in[] = {{q, B * H * S * d * e, "q"},   {k, B * Hk * S * d * e, "k"},
                      {v, B * Hk * S * d * e, "v"},  {lmk, B * Hk * (S / 64) * d * e, "lmk"},
                      {h, qcal ? B * S * D * e : 0, "h"}, {w_down, qcal ? r * D * e : 0, "w_down"},
                      {w_up, qcal ? H * d * r * e : 0, "w_up"}};
  const Range out[] = {{o, B * H * S * d * e, "o"},
                       {sel_idx, with_sel ? B * H * S * kk * 4 : 0, "sel_idx"},
                       {sel_w, with_sel ? B * H * S * kk * 4 : 0, "sel_w"},
                       {workspace, L.total, "workspace"}};
  for (const Range& a : out) {
    for (const Range& b : in)
      if (overlap(a, b)) return fail(HILS_ERR_INVALID_ARG, "%s overlaps input %s", a.name, b.name);
    for (const Range& b : out)
      if (&a != &b && overlap(a, b)) return fail(HILS_ERR_INVALID_ARG, "%s overlaps %s", a.name, b.name);
  }
  char* ws = static_cast<char*>(workspace);
  float* tcode = qcal ? reinterpret_cast<float*>(ws + L.tcode) : nullptr;
  int32_t* idx = with_sel ? sel_idx : reinterpret_cast<int32_t*>(ws + L.idx);
  float* w = with_sel ? sel_w : reinterpret_cast<float*>(ws + L.w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (p->dtype == HILS_DTYPE_BF16) {
    err = p->head_dim == 64
              ? run_prefill<hils::bf16, 64>(p, q, k, v, lmk, h, w_down, w_up, o, idx, w, tcode, ws, L, s)
              : run_prefill<hils::bf16, 128>(p, q, k, v, lmk, h, w_down, w_up, o, idx, w, tcode, ws, L, s);
  } else {
    err = p->head_dim == 64
              ? run_prefill<float, 64>(p, q, k, v, lmk, h, w_down, w_up, o, idx, w, tcode, ws, L, s)
              : run_prefill<float, 128>(p, q, k, v, lmk, h, w_down, w_up, o, idx, w, tcode, ws, L, s);
  }
  if (err != hipSuccess) return hip_fail(err, "hils_prefill_fwd");
  return HILS_OK;
}

int hils_decode_fwd(const hils_decode_params* p, const void* q, const void* k_cache,
                    const void* v_cache, const void* lmk, const int32_t* kv_len, const void* h,
                    const void* w_down, const void* w_up, void* o, int32_t* sel_idx, float* sel_w,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
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
  const size_t N = (Lm + 63) / 64, r = p->qcal_rank, D = p->hidden;
  const size_t Hk = p->kv_heads > 0 ? (size_t)p->kv_heads : H;   // key/value heads
  const size_t cache = p->block_table ? (size_t)p->num_pages * Hk * 64 * d * e : B * Hk * Lm * d * e;
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
  if (p->dtype == HILS_DTYPE_BF16) {
    err = p->head_dim == 64
              ? run_decode<hils::bf16, 64>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s)
              : run_decode<hils::bf16, 128>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s);
  } else {
    err = p->head_dim == 64
              ? run_decode<float, 64>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s)
              : run_decode<float, 128>(p, q, k_cache, v_cache, lmk, kv_len, h, w_down, w_up, o, idx, w, ws, L, s);
  }
  if (err != hipSuccess) return hip_fail(err, "hils_decode_fwd");
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

const char* hils_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
