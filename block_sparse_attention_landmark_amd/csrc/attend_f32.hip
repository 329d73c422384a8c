// Block-sparse attention over the attended block lists: the float32 path (prefill and decode),
// a plain kernel with one query row per lane and float32 arithmetic throughout.  Same PLAIN /
// SAS / HiLS rules as the bf16 kernels.
#include <math.h>

#include <algorithm>

#include "attend_common.hpp"
#include "bsa_internal.hpp"

namespace bsa {

// =============================================================================================
// float32 path (exact-ish reference shapes; one wave, one query row per lane)
// =============================================================================================
// prefill: workgroup per (b, query head, query block), lane = token; decode: workgroup per
// (b, kv group), lane = query head of the group, token = Tk - 1.
template <int D, int MODE>
__global__ __launch_bounds__(64) void attend_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lm, const int32_t* __restrict__ idx, const float* __restrict__ sc,
    float* __restrict__ out, float* __restrict__ lse, int Hq, int Hkv, int G, int Tq, int Tk,
    int NB, int R, int NA, int decode, float scale) {
  __shared__ float Kf[kBlock][D];
  __shared__ float Vf[kBlock][D];
  const int lane = threadIdx.x;
  int b, h, g, c, tq, row_sel;
  bool row_ok;
  if (decode) {
    b = blockIdx.y;
    g = blockIdx.x;
    h = g * G + min(lane, G - 1);
    row_ok = lane < G;
    tq = Tk - 1;
    c = tq / kBlock;
    row_sel = 0;
  } else {
    c = blockIdx.x;
    h = blockIdx.y;
    b = blockIdx.z;
    g = h / G;
    tq = c * kBlock + lane;
    row_ok = tq < Tq;
    row_sel = c;
  }
  const float* qrow = q + ((size_t)(b * Hq + h) * Tq + (decode ? 0 : min(tq, Tq - 1))) * D;
  float qv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = qrow[d];
  const size_t kvbase = (size_t)(b * Hkv + g) * Tk * D;
  const size_t rs = ((size_t)(b * Hkv + g) * R + row_sel) * NA;
  const int nval = count_valid(idx + rs, NA);
  const float s_ref = (MODE == 1 && nval > 0) ? sc[rs + nval - 1] : 0.0f;
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  for (int a = 0; a < nval; ++a) {
    const int j = idx[rs + a];
    if (j < 0 || j > c) continue;
    __syncthreads();
    for (int e = lane; e < kBlock * D; e += 64) {
      const int r = e / D, d = e % D;
      const int tok = j * kBlock + r;
      Kf[r][d] = tok < Tk ? k[kvbase + (size_t)tok * D + d] : 0.0f;
      Vf[r][d] = tok < Tk ? v[kvbase + (size_t)tok * D + d] : 0.0f;
    }
    __syncthreads();
    const float gate = (MODE == 1 && j != c) ? log_sigmoid(sc[rs + a] - s_ref) : 0.0f;
    float s[kBlock];
    float mj = -INFINITY;
    for (int u = 0; u < kBlock; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(qv[d], Kf[u][d], acc);
      const int tok = j * kBlock + u;
      s[u] = (tok <= tq && tok < Tk) ? acc * scale + gate : -INFINITY;
      mj = fmaxf(mj, s[u]);
    }
    float coef = 1.0f, alpha;
    if constexpr (MODE == 2) {
      float lj = 0.0f;
      for (int u = 0; u < kBlock; ++u) {
        s[u] = expf(s[u] - mj);
        lj += s[u];
      }
      const float* lrow = lm + ((size_t)(b * Hkv + g) * NB + j) * D;
      float r = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) r = fmaf(qv[d], lrow[d], r);
      r *= scale;
      const float m_new = fmaxf(m_run, r);
      alpha = expf(m_run - m_new);
      const float wr = expf(r - m_new);
      l_run = l_run * alpha + wr;
      m_run = m_new;
      coef = wr / lj;
    } else {
      const float m_new = fmaxf(m_run, mj);
      alpha = expf(m_run - m_new);
      float lsum = 0.0f;
      for (int u = 0; u < kBlock; ++u) {
        s[u] = expf(s[u] - m_new);
        lsum += s[u];
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
    }
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
    for (int u = 0; u < kBlock; ++u) {
      const float p = s[u] * coef;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vf[u][d], o[d]);
    }
  }
  if (!row_ok) return;
  const size_t orow = decode ? (size_t)(b * Hq + h) : (size_t)(b * Hq + h) * Tq + tq;
#pragma unroll
  for (int d = 0; d < D; ++d) out[orow * D + d] = o[d] / l_run;
  if (MODE != 2 && lse != nullptr) lse[orow] = m_run + logf(l_run);
}

template <int D>
static void launch_f32_d(const Shape& s, const void* q, const void* k, const void* v,
                         const void* lm, const int32_t* idx, const float* sc, void* out,
                         float* lse, hipStream_t st) {
  dim3 grid = s.decode ? dim3(s.Hkv, s.B) : dim3(s.R, s.Hq, s.B);
#define BSA_F32(MODE)                                                                          \
  hipLaunchKernelGGL((attend_f32_kernel<D, MODE>), grid, dim3(64), 0, st, (const float*)q,     \
                     (const float*)k, (const float*)v, (const float*)lm, idx, sc, (float*)out, \
                     lse, s.Hq, s.Hkv, s.G, s.Tq, s.Tk, s.NB, s.R, s.NA, s.decode ? 1 : 0,     \
                     s.scale)
  if (s.mode == 0) BSA_F32(0);
  else if (s.mode == 1) BSA_F32(1);
  else BSA_F32(2);
#undef BSA_F32
}

hipError_t launch_attend_f32(const Shape& s, const void* q, const void* k, const void* v,
                             const void* lm, const int32_t* idx, const float* sc, void* out,
                             float* lse, hipStream_t st) {
  if (s.D == 128) launch_f32_d<128>(s, q, k, v, lm, idx, sc, out, lse, st);
  else launch_f32_d<64>(s, q, k, v, lm, idx, sc, out, lse, st);
  return hipGetLastError();
}

}  // namespace bsa
