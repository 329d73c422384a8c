// C-ABI entry points: argument validation, workspace sizing and kernel dispatch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "bsa.h"
#include "bsa_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

bsa_status_t fail(bsa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bsa_status_t fail(bsa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bsa_status_t ok() {
  g_last_error[0] = '\0';
  return BSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

enum Call { kPool, kSelect, kPrefill, kDecode };

// Validate params for a call and fill the derived shape.
bsa_status_t make_shape(const bsa_params_t* p, Call call, bsa::Shape* s) {
  if (p == nullptr) return fail(BSA_ERR_NULL, "params is NULL");
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->seq_k < 1 || p->seq_q < 1)
    return fail(BSA_ERR_SHAPE, "batch, heads_q, heads_kv, seq_q and seq_k must be >= 1");
  if (p->heads_q % p->heads_kv != 0)
    return fail(BSA_ERR_SHAPE, "heads_q (%d) is not a multiple of heads_kv (%d)", p->heads_q,
                p->heads_kv);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", p->head_dim);
  if (p->block != 64) return fail(BSA_ERR_UNSUPPORTED, "block %d is not 64", p->block);
  if (p->dtype != BSA_DTYPE_F32 && p->dtype != BSA_DTYPE_BF16)
    return fail(BSA_ERR_UNSUPPORTED, "dtype %d is not BSA_DTYPE_F32 or BSA_DTYPE_BF16", p->dtype);
  if (call != kPool) {
    if (p->topk < 0 || p->n_sink < 0 || p->n_local < 1)
      return fail(BSA_ERR_SHAPE, "need topk >= 0, n_sink >= 0, n_local >= 1 (got %d, %d, %d)",
                  p->topk, p->n_sink, p->n_local);
    if ((int64_t)p->topk + p->n_sink + p->n_local > 65536)
      return fail(BSA_ERR_SHAPE, "n_sink + n_local + topk exceeds 65536");
    if (p->seq_q != 1 && p->seq_q != p->seq_k)
      return fail(BSA_ERR_SHAPE, "seq_q (%d) must equal seq_k (%d) for prefill or be 1 for decode",
                  p->seq_q, p->seq_k);
    if (call == kPrefill && p->seq_q != p->seq_k)
      return fail(BSA_ERR_SHAPE, "prefill needs seq_q == seq_k (got %d, %d)", p->seq_q, p->seq_k);
    if (call == kDecode && p->seq_q != 1)
      return fail(BSA_ERR_SHAPE, "decode needs seq_q == 1 (got %d)", p->seq_q);
    if (p->mode < BSA_MODE_PLAIN || p->mode > BSA_MODE_HILS)
      return fail(BSA_ERR_UNSUPPORTED, "mode %d is not PLAIN, SAS or HILS", p->mode);
    if (!(p->scale >= 0.0f) || !isfinite(p->scale))
      return fail(BSA_ERR_SHAPE, "scale must be finite and >= 0 (0 = 1/sqrt(head_dim))");
  }
  // element counts must stay inside what the kernels index with 64-bit offsets and 32-bit
  // block counts
  const int64_t tok_elems = (int64_t)p->batch * p->heads_q * p->seq_k * p->head_dim;
  if (tok_elems > ((int64_t)1 << 40)) return fail(BSA_ERR_SHAPE, "tensor too large");
  bsa::Shape& x = *s;
  x.B = p->batch;
  x.Hq = p->heads_q;
  x.Hkv = p->heads_kv;
  x.G = p->heads_q / p->heads_kv;
  x.D = p->head_dim;
  x.Tk = p->seq_k;
  x.Tq = (call == kPool) ? p->seq_k : p->seq_q;
  // a one-token query against a longer key sequence is a decode step; seq_q == seq_k == 1 is
  // the same computation either way and is treated as prefill by the selection call
  x.decode = (call == kDecode) || (call == kSelect && p->seq_q == 1 && p->seq_k != 1);
  x.NB = (x.Tk + 63) / 64;
  x.R = x.decode ? 1 : (x.Tq + 63) / 64;
  x.c_dec = (x.Tk - 1) / 64;
  x.topk = p->topk;
  x.n_sink = p->n_sink;
  x.n_local = p->n_local;
  x.NA = p->n_sink + p->n_local + p->topk;
  x.mode = p->mode;
  x.bf16 = p->dtype == BSA_DTYPE_BF16;
  x.scale = (p->scale == 0.0f) ? (float)(1.0 / sqrt((double)p->head_dim)) : p->scale;
  if (call == kPrefill || call == kDecode) {
    if (call == kDecode && x.bf16 && x.G > 32)
      return fail(BSA_ERR_UNSUPPORTED, "bf16 decode supports heads_q / heads_kv <= 32 (got %d)", x.G);
  }
  return BSA_OK;
}

bsa_status_t check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(BSA_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(BSA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return BSA_OK;
}

bsa_status_t hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define BSA_TRY(expr)                  \
  do {                                 \
    bsa_status_t st_ = (expr);         \
    if (st_ != BSA_OK) return st_;     \
  } while (0)

// checks shared by the paged (ragged) decode calls
bsa_status_t check_paged(const bsa_params_t* params, const bsa::Shape& s, int32_t n_pages,
                         const int32_t* page_table, const int32_t* seq_lens, bool need_table) {
  if (params->seq_k % 64 != 0)
    return fail(BSA_ERR_SHAPE, "paged calls need seq_k (the capacity) to be a multiple of 64 (got %d)",
                params->seq_k);
  if (need_table) {
    if (n_pages < 1) return fail(BSA_ERR_SHAPE, "n_pages must be >= 1 (got %d)", n_pages);
    BSA_TRY(check_ptr(page_table, "page_table"));
  }
  BSA_TRY(check_ptr(seq_lens, "seq_lens"));
  (void)s;
  return BSA_OK;
}

}  // namespace

extern "C" {

const char* bsa_status_string(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_NULL: return "null pointer";
    case BSA_ERR_SHAPE: return "invalid shape";
    case BSA_ERR_UNSUPPORTED: return "unsupported parameter";
    case BSA_ERR_ALIGN: return "misaligned pointer";
    case BSA_ERR_WORKSPACE: return "workspace too small";
    case BSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* bsa_last_error(void) { return g_last_error; }

int bsa_version(void) { return 100; }

bsa_status_t bsa_pool_landmarks(const bsa_params_t* params, const void* k, void* lm,
                                void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kPool, &s));
  BSA_TRY(check_ptr(k, "k"));
  BSA_TRY(check_ptr(lm, "lm"));
  return hip_result(bsa::launch_pool_landmarks(s, k, lm, (hipStream_t)stream), "pool_landmarks");
}

bsa_status_t bsa_update_landmarks(const bsa_params_t* params, const void* k, int32_t n_new,
                                  void* lm, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kPool, &s));
  if (n_new < 1) return fail(BSA_ERR_SHAPE, "n_new must be >= 1 (got %d)", n_new);
  BSA_TRY(check_ptr(k, "k"));
  BSA_TRY(check_ptr(lm, "lm"));
  return hip_result(bsa::launch_pool_landmarks(s, k, lm, (hipStream_t)stream, n_new),
                    "update_landmarks");
}

size_t bsa_select_workspace_bytes(const bsa_params_t* params) {
  bsa::Shape s;
  if (make_shape(params, kSelect, &s) != BSA_OK) return 0;
  return bsa::select_ws_bytes(s);
}

bsa_status_t bsa_select_topk(const bsa_params_t* params, const void* q, const void* lm,
                             int32_t* idx, float* sc, void* ws, size_t ws_bytes, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kSelect, &s));
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(sc, "sc"));
  const size_t need = bsa::select_ws_bytes(s);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSA_ERR_WORKSPACE, "select workspace needs %zu bytes (got %zu%s)", need,
                  ws_bytes, ws == nullptr ? ", NULL pointer" : "");
    if (((uintptr_t)ws & 255u) != 0) return fail(BSA_ERR_ALIGN, "ws is not 256-byte aligned");
  }
  hipStream_t st = (hipStream_t)stream;
  if (bsa::decode_select_fused(s))
    return hip_result(bsa::launch_decode_select(s, q, lm, idx, sc, st), "select_topk");
  if (bsa::select_fused(s))
    return hip_result(bsa::launch_select_fused(s, q, lm, idx, sc, st), "select_topk");
  float* qbar = (float*)ws;
  hipError_t e = bsa::launch_selector_vectors(s, q, qbar, st);
  float* scores = (float*)((char*)ws + bsa::select_ws_qbar_bytes(s));
  if (e == hipSuccess) e = bsa::launch_block_scores(s, qbar, lm, scores, st);
  if (e == hipSuccess) e = bsa::launch_topk(s, scores, idx, sc, st);
  return hip_result(e, "select_topk");
}

bsa_status_t bsa_select_topk_fused(const bsa_params_t* params, const void* q, const void* lm,
                                   int32_t* idx, float* sc, void* ws, size_t ws_bytes,
                                   void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kSelect, &s));
  if (!bsa::select_fused_ok(s))
    return fail(BSA_ERR_UNSUPPORTED,
                "the one-pass selection takes prefill rows of bf16 landmarks with topk <= 32 and "
                "at most 65536 blocks");
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(sc, "sc"));
  (void)ws;                                    // no workspace: the kernel forms the selector vectors
  (void)ws_bytes;
  return hip_result(bsa::launch_select_fused(s, q, lm, idx, sc, (hipStream_t)stream),
                    "select_topk_fused");
}

bsa_status_t bsa_attend_prefill(const bsa_params_t* params, const void* q, const void* k,
                                const void* v, const void* lm, const int32_t* idx,
                                const float* sc, void* out, float* lse, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kPrefill, &s));
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(k, "k"));
  BSA_TRY(check_ptr(v, "v"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(out, "out"));
  if (s.mode == BSA_MODE_SAS) BSA_TRY(check_ptr(sc, "sc"));
  if (s.mode == BSA_MODE_HILS) {
    BSA_TRY(check_ptr(lm, "lm"));
    if (lse != nullptr) return fail(BSA_ERR_UNSUPPORTED, "lse is not defined for HILS; pass NULL");
  }
  if (lse != nullptr) BSA_TRY(check_ptr(lse, "lse"));
  return hip_result(bsa::launch_attend_prefill(s, q, k, v, lm, idx, sc, out, lse,
                                               (hipStream_t)stream),
                    "attend_prefill");
}

// ---- flat clustered (LSA) index ----

namespace {
bsa_status_t check_lsa_index(int32_t seg_blocks, int32_t n_clusters) {
  if (!bsa::lsa_index_ok(seg_blocks, n_clusters))
    return fail(BSA_ERR_UNSUPPORTED, "need 1 <= n_clusters <= seg_blocks <= 64 (got %d, %d)",
                n_clusters, seg_blocks);
  return BSA_OK;
}

// the flat selection's limits
bsa_status_t check_lsa(const bsa::Shape& s, int32_t seg_blocks, int32_t n_clusters) {
  BSA_TRY(check_lsa_index(seg_blocks, n_clusters));
  if (!bsa::lsa_shape_ok(s, seg_blocks, n_clusters))
    return fail(BSA_ERR_UNSUPPORTED,
                "the LSA selection sorts at most 8192 units per row (segments x n_clusters + "
                "seg_blocks) and chooses at most 2048 blocks (topk)");
  return BSA_OK;
}
}  // namespace

bsa_status_t bsa_lsa_build_index(const bsa_params_t* params, const void* lm, int32_t seg_blocks,
                                 int32_t n_clusters, float* centres, int32_t* members,
                                 int32_t* offsets, int32_t* merges, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kPool, &s));
  BSA_TRY(check_lsa_index(seg_blocks, n_clusters));
  if (s.NB / seg_blocks == 0) return ok();       // no completed segment: nothing to build
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(centres, "centres"));
  BSA_TRY(check_ptr(members, "members"));
  BSA_TRY(check_ptr(offsets, "offsets"));
  if (seg_blocks > n_clusters) BSA_TRY(check_ptr(merges, "merges"));
  return hip_result(bsa::launch_lsa_build(s, lm, seg_blocks, n_clusters, centres, members, offsets,
                                          merges, (hipStream_t)stream),
                    "lsa_build_index");
}

bsa_status_t bsa_lsa_update_index(const bsa_params_t* params, const void* lm, int32_t seg_blocks,
                                  int32_t n_clusters, int32_t first_segment, float* centres,
                                  int32_t* members, int32_t* offsets, int32_t* merges,
                                  void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kPool, &s));
  BSA_TRY(check_lsa_index(seg_blocks, n_clusters));
  if (first_segment < 0)
    return fail(BSA_ERR_SHAPE, "first_segment must be >= 0 (got %d)", first_segment);
  if (s.NB / seg_blocks <= first_segment) return ok();   // no segment to cluster
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(centres, "centres"));
  BSA_TRY(check_ptr(members, "members"));
  BSA_TRY(check_ptr(offsets, "offsets"));
  if (seg_blocks > n_clusters) BSA_TRY(check_ptr(merges, "merges"));
  return hip_result(bsa::launch_lsa_build(s, lm, seg_blocks, n_clusters, centres, members, offsets,
                                          merges, (hipStream_t)stream, first_segment),
                    "lsa_update_index");
}

size_t bsa_lsa_select_workspace_bytes(const bsa_params_t* params) {
  bsa::Shape s;
  if (make_shape(params, kSelect, &s) != BSA_OK) return 0;
  return s.decode ? 0 : bsa::select_ws_qbar_bytes(s) + bsa::lsa_ws_score_bytes(s);
}

bsa_status_t bsa_lsa_select(const bsa_params_t* params, const void* q, const void* lm,
                            int32_t seg_blocks, int32_t n_clusters, const float* centres,
                            const int32_t* members, const int32_t* offsets, int32_t* idx,
                            float* sc, void* ws, size_t ws_bytes, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kSelect, &s));
  BSA_TRY(check_lsa(s, seg_blocks, n_clusters));
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(sc, "sc"));
  if (s.NB / seg_blocks > 0) {
    BSA_TRY(check_ptr(centres, "centres"));
    BSA_TRY(check_ptr(members, "members"));
    BSA_TRY(check_ptr(offsets, "offsets"));
  }
  const size_t need = s.decode ? 0 : bsa::select_ws_qbar_bytes(s);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSA_ERR_WORKSPACE, "LSA selection workspace needs %zu bytes (got %zu%s)", need,
                  ws_bytes, ws == nullptr ? ", NULL pointer" : "");
    if (((uintptr_t)ws & 255u) != 0) return fail(BSA_ERR_ALIGN, "ws is not 256-byte aligned");
  }
  return hip_result(bsa::launch_lsa_select(s, q, lm, seg_blocks, n_clusters, centres, members,
                                           offsets, idx, sc, (float*)ws, ws_bytes,
                                           (hipStream_t)stream),
                    "lsa_select");
}

bsa_status_t bsa_lsa_tree_centres(const bsa_params_t* params, const void* lm,
                                  int32_t seg_blocks, int32_t fanout, float* seg_centres,
                                  float* grp_centres, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kPool, &s));
  if (seg_blocks < 1 || seg_blocks > 64 || fanout < 1)
    return fail(BSA_ERR_UNSUPPORTED, "need 1 <= seg_blocks <= 64 and fanout >= 1 (got %d, %d)",
                seg_blocks, fanout);
  const int ns = s.NB / seg_blocks;
  if (ns == 0) return ok();
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(seg_centres, "seg_centres"));
  if (ns / fanout > 0) BSA_TRY(check_ptr(grp_centres, "grp_centres"));
  return hip_result(bsa::launch_lsa_tree_centres(s, lm, seg_blocks, fanout, seg_centres,
                                                 grp_centres, (hipStream_t)stream),
                    "lsa_tree_centres");
}

bsa_status_t bsa_lsa_tree_select(const bsa_params_t* params, const void* q, const void* lm,
                                 int32_t seg_blocks, int32_t n_clusters, int32_t fanout,
                                 int32_t beam, const float* centres, const int32_t* members,
                                 const int32_t* offsets, const float* seg_centres,
                                 const float* grp_centres, int32_t* idx, float* sc, void* ws,
                                 size_t ws_bytes, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kSelect, &s));
  BSA_TRY(check_lsa_index(seg_blocks, n_clusters));
  if (!bsa::lsa_tree_shape_ok(s, seg_blocks, n_clusters, fanout, beam))
    return fail(BSA_ERR_UNSUPPORTED,
                "the LSA tree needs topk <= 2048, 1 <= beam <= 64, fanout >= 1, and "
                "segments / fanout + fanout, beam * fanout, beam * n_clusters and "
                "beam + seg_blocks at most 1024");
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(sc, "sc"));
  const int ns = s.NB / seg_blocks;
  if (ns > 0) {
    BSA_TRY(check_ptr(centres, "centres"));
    BSA_TRY(check_ptr(members, "members"));
    BSA_TRY(check_ptr(offsets, "offsets"));
    BSA_TRY(check_ptr(seg_centres, "seg_centres"));
    if (ns / fanout > 0) BSA_TRY(check_ptr(grp_centres, "grp_centres"));
  }
  const size_t need = s.decode ? 0 : bsa::select_ws_qbar_bytes(s);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSA_ERR_WORKSPACE, "LSA selection workspace needs %zu bytes (got %zu%s)", need,
                  ws_bytes, ws == nullptr ? ", NULL pointer" : "");
    if (((uintptr_t)ws & 255u) != 0) return fail(BSA_ERR_ALIGN, "ws is not 256-byte aligned");
  }
  return hip_result(bsa::launch_lsa_tree_select(s, q, lm, seg_blocks, n_clusters, fanout, beam,
                                                centres, members, offsets, seg_centres,
                                                grp_centres, idx, sc, (float*)ws,
                                                (hipStream_t)stream),
                    "lsa_tree_select");
}

// ---- backward of PLAIN / SAS prefill ----

namespace {
bsa_status_t backward_shape(const bsa_params_t* params, bsa::Shape* s) {
  BSA_TRY(make_shape(params, kPrefill, s));
  if (!s->bf16) return fail(BSA_ERR_UNSUPPORTED, "the backward pass is implemented for bf16 only");
  if (s->NB > 65535)
    return fail(BSA_ERR_UNSUPPORTED, "the backward pass supports at most 65535 key blocks (got %d)",
                s->NB);
  if ((int64_t)s->R * s->NA >= ((int64_t)1 << 31))
    return fail(BSA_ERR_SHAPE, "query blocks x attended entries exceeds 2^31 - 1");
  return BSA_OK;
}
}  // namespace

size_t bsa_backward_workspace_bytes(const bsa_params_t* params) {
  bsa::Shape s;
  if (backward_shape(params, &s) != BSA_OK) return 0;
  return bsa::backward_ws_bytes(s);
}

bsa_status_t bsa_attend_prefill_backward(const bsa_params_t* params, const void* q,
                                         const void* k, const void* v, const void* lm,
                                         const int32_t* idx, const float* sc, const void* out,
                                         const float* lse, const void* dout, void* dq, void* dk,
                                         void* dv, float* dsc, float* dlm, void* ws,
                                         size_t ws_bytes, void* stream) {
  bsa::Shape s;
  BSA_TRY(backward_shape(params, &s));
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(k, "k"));
  BSA_TRY(check_ptr(v, "v"));
  BSA_TRY(check_ptr(idx, "idx"));
  if (s.mode == BSA_MODE_HILS) {
    BSA_TRY(check_ptr(lm, "lm"));
    BSA_TRY(check_ptr(dlm, "dlm"));
  } else {
    BSA_TRY(check_ptr(out, "out"));
    BSA_TRY(check_ptr(lse, "lse"));
  }
  BSA_TRY(check_ptr(dout, "dout"));
  BSA_TRY(check_ptr(dq, "dq"));
  BSA_TRY(check_ptr(dk, "dk"));
  BSA_TRY(check_ptr(dv, "dv"));
  if (s.mode == BSA_MODE_SAS) {
    BSA_TRY(check_ptr(sc, "sc"));
    BSA_TRY(check_ptr(dsc, "dsc"));
  } else if (dsc != nullptr) {
    BSA_TRY(check_ptr(dsc, "dsc"));
  }
  const size_t need = bsa::backward_ws_bytes(s);
  if (ws == nullptr || ws_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "backward workspace needs %zu bytes (got %zu%s)", need,
                ws_bytes, ws == nullptr ? ", NULL pointer" : "");
  if (((uintptr_t)ws & 255u) != 0) return fail(BSA_ERR_ALIGN, "ws is not 256-byte aligned");
  return hip_result(bsa::launch_attend_backward(s, q, k, v, lm, idx, sc, out, lse, dout, dq, dk,
                                                dv, dsc, s.mode == BSA_MODE_HILS ? dlm : nullptr,
                                                ws, (hipStream_t)stream),
                    "attend_prefill_backward");
}

size_t bsa_decode_workspace_bytes(const bsa_params_t* params) {
  bsa::Shape s;
  if (make_shape(params, kDecode, &s) != BSA_OK) return 0;
  return bsa::decode_ws_bytes(s);
}

bsa_status_t bsa_attend_decode(const bsa_params_t* params, const void* q, const void* kc,
                               const void* vc, const void* lm, const int32_t* idx,
                               const float* sc, void* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kDecode, &s));
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(kc, "kc"));
  BSA_TRY(check_ptr(vc, "vc"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(out, "out"));
  if (s.mode == BSA_MODE_SAS) BSA_TRY(check_ptr(sc, "sc"));
  if (s.mode == BSA_MODE_HILS) {
    BSA_TRY(check_ptr(lm, "lm"));
    if (lse != nullptr) return fail(BSA_ERR_UNSUPPORTED, "lse is not defined for HILS; pass NULL");
  }
  if (lse != nullptr) BSA_TRY(check_ptr(lse, "lse"));
  const size_t need = bsa::decode_ws_bytes(s);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSA_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", need,
                  ws_bytes, ws == nullptr ? ", NULL pointer" : "");
    if (((uintptr_t)ws & 255u) != 0) return fail(BSA_ERR_ALIGN, "ws is not 256-byte aligned");
  }
  return hip_result(bsa::launch_attend_decode(s, q, kc, vc, lm, idx, sc, out, lse, ws,
                                              (hipStream_t)stream),
                    "attend_decode");
}

bsa_status_t bsa_attend_decode_noalloc(const bsa_params_t* params, const void* q, const void* kc,
                                       const void* vc, const void* lm, const int32_t* idx,
                                       const float* sc, void* out, float* lse, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kDecode, &s));
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(kc, "kc"));
  BSA_TRY(check_ptr(vc, "vc"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(out, "out"));
  if (s.mode == BSA_MODE_SAS) BSA_TRY(check_ptr(sc, "sc"));
  if (s.mode == BSA_MODE_HILS) {
    BSA_TRY(check_ptr(lm, "lm"));
    if (lse != nullptr) return fail(BSA_ERR_UNSUPPORTED, "lse is not defined for HILS; pass NULL");
  }
  if (lse != nullptr) BSA_TRY(check_ptr(lse, "lse"));
  const size_t need = bsa::decode_ws_bytes(s);
  if (need > bsa::kNoAllocScratchBytes)
    return fail(BSA_ERR_WORKSPACE,
                "these shapes need %zu bytes of split partials; the static scratch of "
                "bsa_attend_decode_noalloc holds %zu bytes (use bsa_attend_decode with a workspace)",
                need, bsa::kNoAllocScratchBytes);
  hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = bsa::noalloc_scratch(st, &ws);
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "static scratch lookup: %s", hipGetErrorString(e));
  }
  return hip_result(bsa::launch_attend_decode(s, q, kc, vc, lm, idx, sc, out, lse, ws, st),
                    "attend_decode_noalloc");
}

// ---- paged (ragged) decode ----

bsa_status_t bsa_pool_landmarks_paged(const bsa_params_t* params, const void* k_pool,
                                      int32_t n_pages, const int32_t* page_table,
                                      const int32_t* seq_lens, void* lm, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kPool, &s));
  BSA_TRY(check_paged(params, s, n_pages, page_table, seq_lens, true));
  BSA_TRY(check_ptr(k_pool, "k_pool"));
  BSA_TRY(check_ptr(lm, "lm"));
  const bsa::Pages pg{page_table, seq_lens, n_pages};
  return hip_result(bsa::launch_pool_landmarks_paged(s, k_pool, pg, lm, (hipStream_t)stream),
                    "pool_landmarks_paged");
}

bsa_status_t bsa_update_landmarks_paged(const bsa_params_t* params, const void* k_pool,
                                        int32_t n_pages, const int32_t* page_table,
                                        const int32_t* seq_lens, int32_t n_new, void* lm,
                                        void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kPool, &s));
  BSA_TRY(check_paged(params, s, n_pages, page_table, seq_lens, true));
  if (n_new < 1) return fail(BSA_ERR_SHAPE, "n_new must be >= 1 (got %d)", n_new);
  BSA_TRY(check_ptr(k_pool, "k_pool"));
  BSA_TRY(check_ptr(lm, "lm"));
  const bsa::Pages pg{page_table, seq_lens, n_pages};
  return hip_result(
      bsa::launch_pool_landmarks_paged(s, k_pool, pg, lm, (hipStream_t)stream, n_new),
      "update_landmarks_paged");
}

bsa_status_t bsa_select_topk_paged(const bsa_params_t* params, const void* q, const void* lm,
                                   const int32_t* seq_lens, int32_t* idx, float* sc,
                                   void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kDecode, &s));
  BSA_TRY(check_paged(params, s, 1, nullptr, seq_lens, false));
  if (!s.bf16) return fail(BSA_ERR_UNSUPPORTED, "paged selection is implemented for bf16 only");
  if (!bsa::decode_select_fused(s))
    return fail(BSA_ERR_UNSUPPORTED, "paged selection supports at most 16384 blocks per sequence");
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(sc, "sc"));
  const bsa::Pages pg{nullptr, seq_lens, 1};
  return hip_result(bsa::launch_decode_select(s, q, lm, idx, sc, (hipStream_t)stream, &pg),
                    "select_topk_paged");
}

bsa_status_t bsa_attend_decode_paged(const bsa_params_t* params, const void* q,
                                     const void* k_pool, const void* v_pool, int32_t n_pages,
                                     const int32_t* page_table, const int32_t* seq_lens,
                                     const void* lm, const int32_t* idx, const float* sc,
                                     void* out, float* lse, void* ws, size_t ws_bytes,
                                     void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kDecode, &s));
  BSA_TRY(check_paged(params, s, n_pages, page_table, seq_lens, true));
  if (!s.bf16) return fail(BSA_ERR_UNSUPPORTED, "paged decode is implemented for bf16 only");
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(k_pool, "k_pool"));
  BSA_TRY(check_ptr(v_pool, "v_pool"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(out, "out"));
  if (s.mode == BSA_MODE_SAS) BSA_TRY(check_ptr(sc, "sc"));
  if (s.mode == BSA_MODE_HILS) {
    BSA_TRY(check_ptr(lm, "lm"));
    if (lse != nullptr) return fail(BSA_ERR_UNSUPPORTED, "lse is not defined for HILS; pass NULL");
  }
  if (lse != nullptr) BSA_TRY(check_ptr(lse, "lse"));
  const size_t need = bsa::decode_ws_bytes(s);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSA_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", need,
                  ws_bytes, ws == nullptr ? ", NULL pointer" : "");
    if (((uintptr_t)ws & 255u) != 0) return fail(BSA_ERR_ALIGN, "ws is not 256-byte aligned");
  }
  const bsa::Pages pg{page_table, seq_lens, n_pages};
  return hip_result(bsa::launch_attend_decode(s, q, k_pool, v_pool, lm, idx, sc, out, lse, ws,
                                              (hipStream_t)stream, &pg),
                    "attend_decode_paged");
}

// ---- one decode step (selection + attention) ----

size_t bsa_decode_step_workspace_bytes(const bsa_params_t* params) {
  bsa::Shape s;
  if (make_shape(params, kDecode, &s) != BSA_OK) return 0;
  if (bsa::decode_step_fused(s)) return 0;
  const size_t sel = bsa::decode_select_fused(s) ? 0 : bsa::select_ws_bytes(s);
  return ((sel + 255) & ~(size_t)255) + bsa::decode_ws_bytes(s);
}

static bsa_status_t check_decode_step(const bsa::Shape& s, const void* q, const void* kc,
                                      const void* vc, const void* lm, const int32_t* idx,
                                      const float* sc, const void* out, const float* lse,
                                      const void* ws, size_t ws_bytes, size_t need) {
  BSA_TRY(check_ptr(q, "q"));
  BSA_TRY(check_ptr(kc, "k cache"));
  BSA_TRY(check_ptr(vc, "v cache"));
  BSA_TRY(check_ptr(lm, "lm"));
  BSA_TRY(check_ptr(idx, "idx"));
  BSA_TRY(check_ptr(sc, "sc"));
  BSA_TRY(check_ptr(out, "out"));
  if (s.mode == BSA_MODE_HILS && lse != nullptr)
    return fail(BSA_ERR_UNSUPPORTED, "lse is not defined for HILS; pass NULL");
  if (lse != nullptr) BSA_TRY(check_ptr(lse, "lse"));
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSA_ERR_WORKSPACE, "decode step workspace needs %zu bytes (got %zu%s)", need,
                  ws_bytes, ws == nullptr ? ", NULL pointer" : "");
    if (((uintptr_t)ws & 255u) != 0) return fail(BSA_ERR_ALIGN, "ws is not 256-byte aligned");
  }
  return BSA_OK;
}

// the selection and the attention as two launches (shapes the fused kernel does not take)
static hipError_t decode_step_unfused(const bsa::Shape& s, const void* q, const void* kc,
                                      const void* vc, const void* lm, int32_t* idx, float* sc,
                                      void* out, float* lse, void* ws, hipStream_t st,
                                      const bsa::Pages* pg) {
  hipError_t e;
  size_t sel = 0;
  if (bsa::decode_select_fused(s)) {
    const bsa::Pages lens{nullptr, pg ? pg->lens : nullptr, 1};
    e = bsa::launch_decode_select(s, q, lm, idx, sc, st, pg ? &lens : nullptr);
  } else {
    sel = (bsa::select_ws_bytes(s) + 255) & ~(size_t)255;
    float* qbar = (float*)ws;
    float* scores = (float*)((char*)ws + bsa::select_ws_qbar_bytes(s));
    e = bsa::launch_selector_vectors(s, q, qbar, st);
    if (e == hipSuccess) e = bsa::launch_block_scores(s, qbar, lm, scores, st);
    if (e == hipSuccess) e = bsa::launch_topk(s, scores, idx, sc, st);
  }
  if (e != hipSuccess) return e;
  void* dws = bsa::decode_ws_bytes(s) > 0 ? (void*)((char*)ws + sel) : nullptr;
  return bsa::launch_attend_decode(s, q, kc, vc, lm, idx, sc, out, lse, dws, st, pg);
}

bsa_status_t bsa_decode_step(const bsa_params_t* params, const void* q, const void* kc,
                             const void* vc, const void* lm, int32_t* idx, float* sc, void* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kDecode, &s));
  BSA_TRY(check_decode_step(s, q, kc, vc, lm, idx, sc, out, lse, ws, ws_bytes,
                            bsa_decode_step_workspace_bytes(params)));
  hipStream_t st = (hipStream_t)stream;
  if (bsa::decode_step_fused(s))
    return hip_result(
        bsa::launch_decode_step_fused(s, q, kc, vc, lm, idx, sc, out, lse, st, nullptr),
        "decode_step");
  return hip_result(decode_step_unfused(s, q, kc, vc, lm, idx, sc, out, lse, ws, st, nullptr),
                    "decode_step");
}

bsa_status_t bsa_decode_step_paged(const bsa_params_t* params, const void* q,
                                   const void* k_pool, const void* v_pool, int32_t n_pages,
                                   const int32_t* page_table, const int32_t* seq_lens,
                                   const void* lm, int32_t* idx, float* sc, void* out,
                                   float* lse, void* ws, size_t ws_bytes, void* stream) {
  bsa::Shape s;
  BSA_TRY(make_shape(params, kDecode, &s));
  BSA_TRY(check_paged(params, s, n_pages, page_table, seq_lens, true));
  if (!s.bf16) return fail(BSA_ERR_UNSUPPORTED, "paged decode is implemented for bf16 only");
  if (!bsa::decode_select_fused(s))
    return fail(BSA_ERR_UNSUPPORTED, "paged selection supports at most 16384 blocks per sequence");
  BSA_TRY(check_decode_step(s, q, k_pool, v_pool, lm, idx, sc, out, lse, ws, ws_bytes,
                            bsa_decode_step_workspace_bytes(params)));
  hipStream_t st = (hipStream_t)stream;
  const bsa::Pages pg{page_table, seq_lens, n_pages};
  if (bsa::decode_step_fused(s))
    return hip_result(
        bsa::launch_decode_step_fused(s, q, k_pool, v_pool, lm, idx, sc, out, lse, st, &pg),
        "decode_step_paged");
  return hip_result(decode_step_unfused(s, q, k_pool, v_pool, lm, idx, sc, out, lse, ws, st, &pg),
                    "decode_step_paged");
}

size_t bsa_workspace_bytes(const bsa_params_t* params, int which) {
  switch (which) {
    case BSA_WS_SELECT: return bsa_select_workspace_bytes(params);
    case BSA_WS_DECODE: return bsa_decode_workspace_bytes(params);
    case BSA_WS_DECODE_STEP: return bsa_decode_step_workspace_bytes(params);
    case BSA_WS_BACKWARD: return bsa_backward_workspace_bytes(params);
    case BSA_WS_LSA_SELECT: return bsa_lsa_select_workspace_bytes(params);
    default: return 0;
  }
}

}  // extern "C"
