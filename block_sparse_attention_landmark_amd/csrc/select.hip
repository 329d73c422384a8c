// Block scoring and top-K selection.
//
// Scores (SAS page, summary paragraph 1: a light selector scores each unit of context; LSA
// page, "The index stops scanning the whole context", paragraph 2: each contiguous block is
// scored): S[c][j] = qbar_c . L_j for every block j <= c.  With bf16 landmarks the product runs
// on the matrix cores: the float32 selector vector is split into three bf16 terms
// (hi + mid + lo, which together carry its 24 significant bits), so every landmark product is
// exact in the float32 accumulator and only the float32 summation rounds.
//
// Selection (SAS page, summary paragraph 1 and "How to apply": hard top-K; LSA page, first
// section, paragraph 4: the start of the context and a recent window are always added; SAS
// page, summary paragraph 3: the current block is always kept): among the candidate blocks
// n_sink <= j <= c - n_local, take the K highest scores, lower block index first among equal
// scores, via a 4-pass 8-bit radix select on order-preserving score keys followed by an
// index-ordered compaction.  The attended set is written ascending: sink blocks, the chosen
// candidates, then the local window ending at c; padding is -1.
#include "bsa_common.hpp"
#include "bsa_internal.hpp"
#include "select_common.hpp"

namespace bsa {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline size_t tri(size_t n) { return n * (n + 1) / 2; }

size_t select_ws_qbar_bytes(const Shape& s) {
  return align256((size_t)s.B * s.Hkv * s.R * s.D * sizeof(float));
}
size_t select_ws_scores_bytes(const Shape& s) {
  const size_t per = s.decode ? (size_t)s.NB : tri((size_t)s.R);
  return align256((size_t)s.B * s.Hkv * per * sizeof(float));
}
size_t select_ws_bytes(const Shape& s) { return select_ws_qbar_bytes(s) + select_ws_scores_bytes(s); }

// ---------------------------------------------------------------------------------------------
// decode scores, bf16 landmarks: the one selection row of each (sequence, kv group) against
// blocks 0..c_dec, 64 blocks per workgroup (tile tj = blockIdx.x), one 32x32 MFMA sub-tile per
// wave (waves 2, 3 hold only padding rows and leave).  Used when the fused decode selection does
// not apply (more than 16384 blocks); prefill rows use score_strip_kernel below.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void score_mfma_kernel(const float* __restrict__ qbar,
                                                         const bf16* __restrict__ lm,
                                                         float* __restrict__ scores, int R,
                                                         int NB, int c_dec) {
  const int bg = blockIdx.y;
  const int tj = blockIdx.x;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const int row0 = (w / 2) * 32;              // R == 1: rows past it are padding
  const int col0 = tj * 64 + (w % 2) * 32;
  if (row0 >= R) return;
  if (col0 > c_dec || col0 >= NB) return;

  const int r = row0 + l32;
  const int j = col0 + l32;
  const float* qrow = qbar + ((size_t)bg * R + min(r, R - 1)) * D;
  const bf16* lrow = lm + ((size_t)bg * NB + min(j, NB - 1)) * D;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int d0 = 16 * s + 8 * half;
    bf16x8 hi, mid, lo, bl;
    f32x4 x0 = *reinterpret_cast<const f32x4*>(qrow + d0);
    f32x4 x1 = *reinterpret_cast<const f32x4*>(qrow + d0 + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = (e < 4) ? x0[e] : x1[e - 4];
      if (r >= R) x = 0.0f;
      const bf16 h = f2bf(x);
      const float r1 = x - bf2f(h);          // exact in float32
      const bf16 m = f2bf(r1);
      hi[e] = h;
      mid[e] = m;
      lo[e] = f2bf(r1 - bf2f(m));            // the remaining <= 8 significant bits
    }
    u32x4 lraw = *reinterpret_cast<const u32x4*>(lrow + d0);
    bl = __builtin_bit_cast(bf16x8, lraw);
    if (j >= NB) {
#pragma unroll
      for (int e = 0; e < 8; ++e) bl[e] = f2bf(0.0f);
    }
    acc = mfma32(hi, bl, acc);
    acc = mfma32(mid, bl, acc);
    acc = mfma32(lo, bl, acc);
  }
  if (j >= NB || j > c_dec) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rr = row0 + 8 * (i / 4) + 4 * half + (i % 4);
    if (rr < R) scores[(size_t)bg * NB + j] = acc[i];
  }
}

// scores of a prefill, bf16 landmarks: one workgroup per strip of up to kScoreStrip column
// tiles (64 x 64) of one tile row of the lower triangle.  Each wave splits the selector vectors
// of its 32 rows into their three bf16 terms once and reuses them for every tile of the strip
// (same products and summation order as score_mfma_kernel, so the scores are identical).
// Strip index p: the tile rows form bands of kScoreStrip rows; the rows of band k hold k + 1
// strips each, so band k starts at strip kScoreStrip * k (k + 1) / 2.
constexpr int kScoreStrip = 8;

template <int D>
__global__ __launch_bounds__(256) void score_strip_kernel(const float* __restrict__ qbar,
                                                          const bf16* __restrict__ lm,
                                                          float* __restrict__ scores, int R,
                                                          int NB) {
  constexpr int S = kScoreStrip;
  const int bg = blockIdx.y;
  const long p = blockIdx.x;
  long k = (long)((sqrt(8.0 * (double)(p / S) + 1.0) - 1.0) * 0.5);
  while ((long)S * (long)tri(k + 1) <= p) ++k;
  while ((long)S * (long)tri(k) > p) --k;
  const long rem = p - (long)S * (long)tri(k);
  const int ti = (int)(k * S + rem / (k + 1));
  const int strip = (int)(rem % (k + 1));
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const int row0 = ti * 64 + (w / 2) * 32;
  if (row0 >= R) return;
  const int last_row = min(row0 + 31, R - 1);
  const int r = row0 + l32;
  const float* qrow = qbar + ((size_t)bg * R + min(r, R - 1)) * D;
  bf16x8 hi[D / 16], mid[D / 16], lo[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const int d0 = 16 * st + 8 * half;
    f32x4 x0 = *reinterpret_cast<const f32x4*>(qrow + d0);
    f32x4 x1 = *reinterpret_cast<const f32x4*>(qrow + d0 + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = (e < 4) ? x0[e] : x1[e - 4];
      if (r >= R) x = 0.0f;
      const bf16 h = f2bf(x);
      const float r1 = x - bf2f(h);          // exact in float32
      const bf16 m = f2bf(r1);
      hi[st][e] = h;
      mid[st][e] = m;
      lo[st][e] = f2bf(r1 - bf2f(m));        // the remaining <= 8 significant bits
    }
  }
  const size_t obase = (size_t)bg * tri(R);
  // landmark fragments of column tile tj (rows past NB read as zeros); the next tile's are
  // loaded while the current one is multiplied
  auto load_l = [&](int tj, bf16x8* bl) {
    const int j = tj * 64 + (w % 2) * 32 + l32;
    const bf16* lrow = lm + ((size_t)bg * NB + min(j, NB - 1)) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      bl[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lrow + 16 * st + 8 * half));
      if (j >= NB) {
#pragma unroll
        for (int e = 0; e < 8; ++e) bl[st][e] = f2bf(0.0f);
      }
    }
  };
  const int tj_end = min(strip * S + S, ti + 1);
  bf16x8 bl[D / 16], bn[D / 16];
  load_l(strip * S, bl);
  for (int tj = strip * S; tj < tj_end; ++tj) {
    const int col0 = tj * 64 + (w % 2) * 32;
    if (col0 > last_row || col0 >= NB) break;
    const int j = col0 + l32;
    if (tj + 1 < tj_end) load_l(tj + 1, bn);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      acc = mfma32(hi[st], bl[st], acc);
      acc = mfma32(mid[st], bl[st], acc);
      acc = mfma32(lo[st], bl[st], acc);
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) bl[st] = bn[st];
    if (j >= NB) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = row0 + 8 * (i / 4) + 4 * half + (i % 4);
      if (rr >= R || j > rr) continue;
      scores[obase + tri(rr) + j] = acc[i];
    }
  }
}

// scores, float32 landmarks: one thread per (row, block), float64 accumulation
template <int D>
__global__ __launch_bounds__(256) void score_f32_kernel(const float* __restrict__ qbar,
                                                        const float* __restrict__ lm,
                                                        float* __restrict__ scores, int R,
                                                        int NB, int c_dec) {
  const int r = blockIdx.y;
  const int bg = blockIdx.z;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int c = (c_dec >= 0) ? c_dec : r;
  if (j > c || j >= NB) return;
  const float* qrow = qbar + ((size_t)bg * R + r) * D;
  const float* lrow = lm + ((size_t)bg * NB + j) * D;
  double acc = 0.0;
#pragma unroll 8
  for (int d = 0; d < D; ++d) acc += (double)qrow[d] * (double)lrow[d];
  const size_t off = (c_dec >= 0) ? (size_t)bg * NB : (size_t)bg * tri(R) + tri(r);
  scores[off + j] = (float)acc;
}

hipError_t launch_block_scores(const Shape& s, const float* qbar, const void* lm, float* scores,
                               hipStream_t st) {
  const int c_dec = s.decode ? s.c_dec : -1;
  if (s.bf16) {
    if (!s.decode) {
      const size_t bands = ((s.R + 63) / 64 + kScoreStrip - 1) / kScoreStrip;
      const dim3 grid((unsigned)(kScoreStrip * tri(bands)), s.B * s.Hkv);
      if (s.D == 128)
        hipLaunchKernelGGL(score_strip_kernel<128>, grid, dim3(256), 0, st, qbar,
                           (const bf16*)lm, scores, s.R, s.NB);
      else
        hipLaunchKernelGGL(score_strip_kernel<64>, grid, dim3(256), 0, st, qbar,
                           (const bf16*)lm, scores, s.R, s.NB);
      return hipGetLastError();
    }
    const dim3 grid((s.c_dec + 1 + 63) / 64, s.B * s.Hkv);
    if (s.D == 128)
      hipLaunchKernelGGL(score_mfma_kernel<128>, grid, dim3(256), 0, st, qbar, (const bf16*)lm,
                         scores, s.R, s.NB, c_dec);
    else
      hipLaunchKernelGGL(score_mfma_kernel<64>, grid, dim3(256), 0, st, qbar, (const bf16*)lm,
                         scores, s.R, s.NB, c_dec);
  } else {
    const int maxc = s.decode ? s.c_dec : s.R - 1;
    dim3 grid((maxc + 1 + 255) / 256, s.R, s.B * s.Hkv);
    if (s.D == 128)
      hipLaunchKernelGGL(score_f32_kernel<128>, grid, dim3(256), 0, st, qbar, (const float*)lm,
                         scores, s.R, s.NB, c_dec);
    else
      hipLaunchKernelGGL(score_f32_kernel<64>, grid, dim3(256), 0, st, qbar, (const float*)lm,
                         scores, s.R, s.NB, c_dec);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// top-K rows from the score workspace (the row select itself: topk_select in select_common.hpp)
// ---------------------------------------------------------------------------------------------
// one workgroup of NT threads per selection row, scores from the score workspace: the row is
// read with 16 loads in flight per thread into an LDS cache of CACHE keys (longer rows re-read
// L2), from which each thread takes its contiguous slice of up to KPT keys into registers.  Rows
// of up to 4096 candidates take 256 threads holding 8 keys each (more rows share a CU; rows of
// 2049..4096 candidates count from LDS), longer ones 1024 threads holding 16, so that every key
// of a row up to 16384 candidates stays in a register through the radix passes; their digit
// counts are spread over 4 words per digit.
template <int CACHE, int NT, int KPT, int REP>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores,
                                                  int32_t* __restrict__ idx,
                                                  float* __restrict__ sc, int R, int NB,
                                                  int c_dec, int topk, int n_sink, int n_local,
                                                  int NA) {
  __shared__ uint32_t skeys[CACHE];
  __shared__ int hist[kTopkHistWords * REP];
  __shared__ int sbuf[NT / kWave];
  __shared__ int sh[2];
  const int r = blockIdx.x;
  const int bg = blockIdx.y;
  const int c = (c_dec >= 0) ? c_dec : r;
  const float* srow = scores + ((c_dec >= 0) ? (size_t)bg * NB : (size_t)bg * tri(R) + tri(c));
  const int n = max(0, c - n_local - n_sink + 1);
  const bool cached = n <= CACHE;
  if (cached) {
    constexpr int U = 16;
    for (int i0 = 0; i0 < n; i0 += NT * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NT + threadIdx.x;
        v[u] = i < n ? srow[n_sink + i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NT + threadIdx.x;
        if (i < n) skeys[i] = float_key(v[u]);
      }
    }
  }
  __syncthreads();
  topk_select<NT, KPT, REP>(
      [&](int j) { return srow[j]; },
      [&](int i) { return cached ? skeys[i] : float_key(srow[n_sink + i]); }, c, topk, n_sink,
      n_local, NA, idx + ((size_t)bg * R + r) * NA, sc + ((size_t)bg * R + r) * NA, hist, sbuf,
      sh);
}

// ---------------------------------------------------------------------------------------------
// decode: selector vector, scores of every block and top-K in one workgroup per (sequence, kv
// group); the landmark rows are read with 16 lanes per row (coalesced 1 KB per instruction)
// ---------------------------------------------------------------------------------------------
constexpr int kDecodeSelThreads = 1024;
constexpr int kDecodeSelMaxBlocks = 16384;    // scores kept in LDS (64 KB)

// (PAGED: sequence b holds seq_lens[b] tokens, clamped to 1 .. NB * 64, and its query is the
// last of them; otherwise every sequence's query block is c_all.)
template <int D, bool PAGED>
__global__ __launch_bounds__(kDecodeSelThreads) void decode_select_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ lm, int32_t* __restrict__ idx,
    float* __restrict__ sc, int Hq, int Hkv, int G, int NB, int c_all, int topk, int n_sink,
    int n_local, int NA, const int32_t* __restrict__ seq_lens) {
  constexpr int LPR = D / 8;                  // lanes per landmark row (8 elements each)
  constexpr int RPI = kWave / LPR;            // rows per wave instruction
  constexpr int NW = kDecodeSelThreads / kWave;
  __shared__ float qb[D];
  __shared__ float ssc[kDecodeSelMaxBlocks];
  __shared__ int hist[kTopkHistWords];
  __shared__ int sbuf[NW];
  __shared__ int sh[2];
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int c = PAGED ? (min(max(seq_lens[b], 1), NB * kBlock) - 1) / kBlock : c_all;
  const int tid = threadIdx.x;
  if (tid < D) {
    double acc = 0.0;
    for (int hh = 0; hh < G; ++hh) acc += (double)bf2f(q[(size_t)(b * Hq + g * G + hh) * D + tid]);
    qb[tid] = (float)acc;
  }
  __syncthreads();
  const int w = tid / kWave, lane = tid % kWave;
  const int part = lane % LPR, sub = lane / LPR;
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qb[part * 8 + e];
  const bf16* lbase = lm + (size_t)bg * NB * D;
  for (int j0 = w * RPI; j0 <= c; j0 += NW * RPI * 4) {
    float acc[4];
    u32x4 raw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(j0 + u * NW * RPI + sub, c);
      raw[u] = *reinterpret_cast<const u32x4*>(lbase + (size_t)j * D + part * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bf16x8 lv = __builtin_bit_cast(bf16x8, raw[u]);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(qv[e], bf2f(lv[e]), s);
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
      acc[u] = s;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * NW * RPI + sub;
      if (part == 0 && j <= c) ssc[j] = acc[u];
    }
  }
  __syncthreads();
  topk_select<kDecodeSelThreads>(
      [&](int j) { return ssc[j]; }, [&](int i) { return float_key(ssc[n_sink + i]); }, c, topk,
      n_sink, n_local, NA, idx + (size_t)bg * NA, sc + (size_t)bg * NA, hist, sbuf, sh);
}

bool decode_select_fused(const Shape& s) {
  return s.decode && s.bf16 && s.c_dec + 1 <= kDecodeSelMaxBlocks;
}

hipError_t launch_decode_select(const Shape& s, const void* q, const void* lm, int32_t* idx,
                                float* sc, hipStream_t st, const Pages* pg) {
  dim3 grid(s.B * s.Hkv);
#define BSA_DSEL(D_, P_)                                                                        \
  hipLaunchKernelGGL((decode_select_bf16_kernel<D_, P_>), grid, dim3(kDecodeSelThreads), 0, st, \
                     (const bf16*)q, (const bf16*)lm, idx, sc, s.Hq, s.Hkv, s.G, s.NB, s.c_dec, \
                     s.topk, s.n_sink, s.n_local, s.NA, pg ? pg->lens : nullptr)
  if (s.D == 128) {
    if (pg) BSA_DSEL(128, true);
    else BSA_DSEL(128, false);
  } else {
    if (pg) BSA_DSEL(64, true);
    else BSA_DSEL(64, false);
  }
#undef BSA_DSEL
  return hipGetLastError();
}

hipError_t launch_topk(const Shape& s, const float* scores, int32_t* idx, float* sc,
                       hipStream_t st) {
  dim3 grid(s.R, s.B * s.Hkv);
  if (s.NB <= 4096)
    hipLaunchKernelGGL((topk_kernel<4096, 256, 8, 1>), grid, dim3(256), 0, st, scores, idx, sc, s.R,
                       s.NB, s.decode ? s.c_dec : -1, s.topk, s.n_sink, s.n_local, s.NA);
  else
    hipLaunchKernelGGL((topk_kernel<16384, 1024, 16, 4>), grid, dim3(1024), 0, st, scores, idx, sc,
                       s.R, s.NB, s.decode ? s.c_dec : -1, s.topk, s.n_sink, s.n_local, s.NA);
  return hipGetLastError();
}

}  // namespace bsa
