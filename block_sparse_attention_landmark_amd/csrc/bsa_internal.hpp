// Internal (C++) interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsa {

// Validated sizes of one call, derived from bsa_params_t.
struct Shape {
  int B, Hq, Hkv, G, D;
  int Tq, Tk;       // query tokens (prefill: == Tk; decode: 1) and key tokens
  int NB;           // key blocks: ceil(Tk / 64)
  int R;            // selection rows per (b, kv group): prefill ceil(Tq / 64), decode 1
  int c_dec;        // decode: block of the query token (Tk - 1) / 64
  int topk, n_sink, n_local, NA;
  int mode;         // 0 plain, 1 sas, 2 hils
  bool bf16, decode;
  float scale;      // softmax scale (already defaulted to 1/sqrt(D))
};

// Paged decode cache: block j of sequence b is page table[b * NB + j] of a pool of n_pages
// 64-token pages [n_pages, Hkv, 64, D]; sequence b holds lens[b] tokens (device pointers).
struct Pages {
  const int32_t* table;
  const int32_t* lens;
  int n_pages;
};

// Block index of selection row r (prefill: r; decode: the query token's block).
inline int row_block(const Shape& s, int r) { return s.decode ? s.c_dec : r; }

// Workspace of bsa_select_topk: selector vectors then scores, each 256-byte aligned.
size_t select_ws_qbar_bytes(const Shape& s);
size_t select_ws_scores_bytes(const Shape& s);
size_t select_ws_bytes(const Shape& s);
// Workspace of bsa_attend_decode: split partials.
int decode_splits(const Shape& s);
size_t decode_ws_bytes(const Shape& s);
// Static per-device scratch that bsa_attend_decode_noalloc uses in place of the workspace: its
// size, and its device address on the device of stream st (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(hipStream_t st, void** ptr);

// n_new > 0: only the blocks holding the last n_new tokens (of every sequence)
hipError_t launch_pool_landmarks(const Shape& s, const void* k, void* lm, hipStream_t st,
                                 int n_new = 0);
hipError_t launch_selector_vectors(const Shape& s, const void* q, float* qbar, hipStream_t st);
hipError_t launch_block_scores(const Shape& s, const float* qbar, const void* lm, float* scores,
                               hipStream_t st);
// Prefill rows of bf16 landmarks with K <= 32: scores and top-K in one kernel, no score workspace
// (select_fused_ok: the kernel applies; select_fused: bsa_select_topk uses it).
bool select_fused_ok(const Shape& s);
bool select_fused(const Shape& s);
hipError_t launch_select_fused(const Shape& s, const void* q, const void* lm, int32_t* idx,
                               float* sc, hipStream_t st);
hipError_t launch_topk(const Shape& s, const float* scores, int32_t* idx, float* sc,
                       hipStream_t st);
// decode with bf16 landmarks: selector vector, scores and top-K in one kernel
bool decode_select_fused(const Shape& s);
hipError_t launch_decode_select(const Shape& s, const void* q, const void* lm, int32_t* idx,
                                float* sc, hipStream_t st, const Pages* pg = nullptr);
hipError_t launch_pool_landmarks_paged(const Shape& s, const void* k_pool, const Pages& pg,
                                       void* lm, hipStream_t st, int n_new = 0);
hipError_t launch_attend_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                 const void* lm, const int32_t* idx, const float* sc, void* out,
                                 float* lse, hipStream_t st);
// float32 path of both attend calls
hipError_t launch_attend_f32(const Shape& s, const void* q, const void* k, const void* v,
                             const void* lm, const int32_t* idx, const float* sc, void* out,
                             float* lse, hipStream_t st);
// one decode step in one kernel per (sequence, kv group): selection, then attention
bool decode_step_fused(const Shape& s);
hipError_t launch_decode_step_fused(const Shape& s, const void* q, const void* kc, const void* vc,
                                    const void* lm, int32_t* idx, float* sc, void* out,
                                    float* lse, hipStream_t st, const Pages* pg);
hipError_t launch_attend_decode(const Shape& s, const void* q, const void* kc, const void* vc,
                                const void* lm, const int32_t* idx, const float* sc, void* out,
                                float* lse, void* ws, hipStream_t st, const Pages* pg = nullptr);

// Backward of bf16 prefill attention (PLAIN / SAS / HiLS): workspace size and launcher.
size_t backward_ws_bytes(const Shape& s);
hipError_t launch_attend_backward(const Shape& s, const void* q, const void* k, const void* v,
                                  const void* lm, const int32_t* idx, const float* sc,
                                  const void* out, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, float* dsc, float* dlm, void* ws,
                                  hipStream_t st);

// Flat clustered (LSA) index: shape limits, index build, selection over it.
bool lsa_index_ok(int seg, int nc);
bool lsa_shape_ok(const Shape& s, int seg, int nc);
// segments seg0 .. NB / seg - 1 (seg0 > 0: only the segments completed since an earlier build)
hipError_t launch_lsa_build(const Shape& s, const void* lm, int seg, int nc, float* centres,
                            int32_t* members, int32_t* offsets, int32_t* merges, hipStream_t st,
                            int seg0 = 0);
size_t lsa_ws_score_bytes(const Shape& s);
hipError_t launch_lsa_select(const Shape& s, const void* q, const void* lm, int seg, int nc,
                             const float* centres, const int32_t* members,
                             const int32_t* offsets, int32_t* idx, float* sc, float* qbar,
                             size_t ws_bytes, hipStream_t st);

// LSA tree index: shape limits, node centres, beam-search selection.
bool lsa_tree_shape_ok(const Shape& s, int seg, int nc, int fan, int beam);
hipError_t launch_lsa_tree_centres(const Shape& s, const void* lm, int seg, int fan, float* seg_c,
                                   float* grp_c, hipStream_t st);
hipError_t launch_lsa_tree_select(const Shape& s, const void* q, const void* lm, int seg, int nc,
                                  int fan, int beam, const float* centres, const int32_t* members,
                                  const int32_t* offsets, const float* seg_c, const float* grp_c,
                                  int32_t* idx, float* sc, float* qbar, hipStream_t st);

}  // namespace bsa
