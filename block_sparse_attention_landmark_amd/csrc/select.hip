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
bool select_fused(const Shape& s);
__host__ __device__ inline size_t tri(size_t n) { return n * (n + 1) / 2; }

size_t select_ws_qbar_bytes(const Shape& s) {
  return align256((size_t)s.B * s.Hkv * s.R * s.D * sizeof(float));
}
size_t select_ws_scores_bytes(const Shape& s) {
  const size_t per = s.decode ? (size_t)s.NB : tri((size_t)s.R);
  return align256((size_t)s.B * s.Hkv * per * sizeof(float));
}
size_t select_ws_bytes(const Shape& s) {
  if (select_fused(s)) return 0;                 // the one-pass kernel needs no workspace
  return select_ws_qbar_bytes(s) + select_ws_scores_bytes(s);
}

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
// prefill selection in one pass (bf16 landmarks, K <= 32): scores and top-K without the score
// workspace.  One workgroup per (tile row of 64 query blocks, batch and kv group); its four
// waves split every 64 x 64 score tile as score_strip_kernel does (same products in the same
// order, so the same scores) and sweep the tile row's column tiles left to right.  Each (row,
// column half) keeps in LDS a list of candidates, appended in block order, and a threshold key:
// a candidate is appended only if its key is above the threshold, the K-th best key among the
// candidates that column half has already seen.  That drops only candidates with K better ones
// seen before them (on equal keys the earlier, lower block wins), which cannot be chosen.  A list
// that could overflow at the next tile is cut to its K best and the threshold raised to its K-th
// key.  At the end the two halves' lists of a row are merged in block order and cut to K.  The
// forced entries (sinks, local window) and the rows whose candidates are all taken are written
// while sweeping, the padding at the end: the same attended sets as topk_select writes.
// ---------------------------------------------------------------------------------------------
constexpr int kFusedCap = 96;        // list slots per (row, column half); a tile appends <= 32
constexpr int kFusedMaxK = 32;

// x from the lane jj apart within each group of 32 lanes (jj = 1, 2, 4, 8, 16)
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x, int jj) {
  const int v = (int)x;
  switch (jj) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, false);   // quad_perm 1,0,3,2
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, false);   // quad_perm 2,3,0,1
    case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle(v, 0x1F | (4 << 10));
    case 8: return (uint32_t)__builtin_amdgcn_ds_swizzle(v, 0x1F | (8 << 10));
    default: return (uint32_t)__builtin_amdgcn_ds_swizzle(v, 0x1F | (16 << 10));
  }
}

// Cut a list of n <= 128 entries (scores ls[0..n), blocks lj[0..n)) to its K best by (key
// descending, slot ascending), keeping their slot order; returns the K-th best key.  One list per
// half-wave (l = lane % 32): both halves of a wave call it together, each with its own list, n
// and K (1 <= K <= 32).  A list of n <= K entries is left as it is (the return value is then
// meaningless).  Slot order is block order for every list cut here.
__device__ __forceinline__ uint32_t cut_list(float* ls, uint16_t* lj, int n, int K, int l) {
  float v[4];
  int jv[4];
  uint32_t key[4], x[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int slot = 32 * s + l;
    const bool in = slot < n;
    v[s] = in ? ls[slot] : 0.0f;
    jv[s] = in ? (int)lj[slot] : 0;
    key[s] = in ? float_key(v[s]) : 0u;    // empty slots sort last (no score has key 0)
    x[s] = key[s];
  }
  // bitonic sort of the 128 keys, descending; element e = 32 s + l
#pragma unroll
  for (int k = 2; k <= 128; k <<= 1) {
#pragma unroll
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj >= 32) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int t = s ^ (jj >> 5);
          if (t > s) {
            const bool desc = ((32 * s + l) & k) == 0;
            const uint32_t mx = max(x[s], x[t]), mn = min(x[s], x[t]);
            x[s] = desc ? mx : mn;
            x[t] = desc ? mn : mx;
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t y = lane_xor32(x[s], jj);
          const bool desc = ((32 * s + l) & k) == 0;
          const bool lower = (l & jj) == 0;
          x[s] = (lower == desc) ? max(x[s], y) : min(x[s], y);
        }
      }
    }
  }
  const int lane = threadIdx.x % kWave;
  const uint32_t tau = (uint32_t)__shfl((int)x[0], (lane & 32) + K - 1, kWave);
  if (n <= K) return tau;
  // keep every key above tau and the first (K - #above) equal to it, in slot order
  const uint32_t below = (1u << l) - 1u;
  const int hshift = lane & 32;
  int n_gt = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    n_gt += __popcll(__ballot(key[s] > tau) >> hshift & 0xffffffffull);
  const int need_eq = K - n_gt;
  int eq_before = 0, pos_base = 0;
  bool keep[4];
  int pos[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bool eq = key[s] == tau && 32 * s + l < n;
    const uint32_t eqm = (uint32_t)(__ballot(eq) >> hshift);
    const int eq_rank = eq_before + __popc(eqm & below);
    keep[s] = key[s] > tau || (eq && eq_rank < need_eq);
    eq_before += __popc(eqm);
    const uint32_t km = (uint32_t)(__ballot(keep[s]) >> hshift);
    pos[s] = pos_base + __popc(km & below);
    pos_base += __popc(km);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s)
    if (keep[s]) {
      ls[pos[s]] = v[s];
      lj[pos[s]] = (uint16_t)jv[s];
    }
  return tau;
}

template <int D>
__global__ __launch_bounds__(256, 2) void select_fused_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ lm, int32_t* __restrict__ idx,
    float* __restrict__ sc, int Hq, int Hkv, int G, int T, int R, int NB, int topk, int n_sink,
    int n_local, int NA) {
  constexpr int CAP = kFusedCap;
  __shared__ float ls[64][2 * CAP];          // per row: column half h in slots h*CAP ..
  __shared__ uint16_t lj[64][2 * CAP];
  __shared__ int lcnt[64][2];
  __shared__ float ltau[64][2];
  // Workgroups are dealt round-robin over the 8 XCDs; with a multiple of 8 (batch, kv group)
  // pairs, XCD x takes the pairs x, x + 8, .. so that each XCD's L2 serves one pair's landmarks
  // at a time.  Heavy (long) tile rows first.
  const int nT = (R + 63) / 64;
  const int n_bg = (int)gridDim.y;
  const int lin = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  int bg, tr;
  if (n_bg % 8 == 0) {
    const int k = lin / 8;
    bg = (k / nT) * 8 + lin % 8;
    tr = k % nT;
  } else {
    bg = lin / nT;
    tr = lin % nT;
  }
  const int ti = nT - 1 - tr;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const int rh = w / 2, ch = w % 2;
  const int row0 = ti * 64 + rh * 32;
  const int last_row = min(row0 + 31, R - 1);
  int32_t* oidx = idx + (size_t)bg * R * NA;
  float* osc = sc + (size_t)bg * R * NA;
  auto lrow = [&](int i) { return rh * 32 + 8 * (i / 4) + 4 * half + (i % 4); };

  // threshold score per (row, column half), uniform in a half-wave: a candidate is appended only
  // if its score is above it (on scores, float order is the key order)
  f32x16 tau;
#pragma unroll
  for (int i = 0; i < 16; ++i) tau[i] = -INFINITY;
  if (l32 == 0) {                              // each wave owns the counts of its lists
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      lcnt[lrow(i)][ch] = 0;
      ltau[lrow(i)][ch] = -INFINITY;
    }
  }

  // Selector vectors of the tile row's 64 query blocks, staged in the (not yet used) list space:
  // for each block, the sum over the group's query heads of the mean over its tokens,
  // accumulated in float64 and rounded once to float32, as the selector pass computes them.
  float* sq = &ls[0][0];
  static_assert(64 * D * sizeof(float) <= sizeof(ls), "selector vectors fit the list space");
  {
    constexpr int NC = D / 8;                  // 16-byte chunks of a row
    constexpr int RS = 256 / NC;               // query blocks in flight per workgroup
    constexpr int U = 32;                      // token rows loaded per batch
    const int tid = threadIdx.x;
    const int cc = tid % NC;
    const int b = bg / Hkv, g = bg % Hkv;
    for (int rl = tid / NC; rl < 64; rl += RS) {
      const int qb = ti * 64 + rl;
      double acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0;
      int ntok = 1;
      if (qb < R) {
        const int t0 = qb * kBlock;
        ntok = min(kBlock, T - t0);
        const int nrows = G * ntok;              // (head, token) rows of the block
        for (int i0 = 0; i0 < nrows; i0 += U) {
          u32x4 raw[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int i = min(i0 + u, nrows - 1);
            const int hh = i / ntok, t = t0 + i % ntok;
            raw[u] = *reinterpret_cast<const u32x4*>(
                q + ((size_t)(b * Hq + g * G + hh) * T + t) * D + cc * 8);
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (i0 + u < nrows) {
              const bf16x8 x = __builtin_bit_cast(bf16x8, raw[u]);
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[e] += (double)bf2f(x[e]);
            }
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sq[rl * D + cc * 8 + e] = qb < R ? (float)(acc[e] / (double)ntok) : 0.0f;
    }
  }
  __syncthreads();

  // each wave splits the selector vectors of its 32 rows into their three bf16 terms
  bf16x8 hi[D / 16], mid[D / 16], lo[D / 16];
  {
    const int r = row0 + l32;
    const float* qrow = sq + (rh * 32 + l32) * D;
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
        const float r1 = x - bf2f(h);        // exact in float32
        const bf16 m = f2bf(r1);
        hi[st][e] = h;
        mid[st][e] = m;
        lo[st][e] = f2bf(r1 - bf2f(m));      // the remaining <= 8 significant bits
      }
    }
  }
  __syncthreads();                             // the list space is free again

  if (row0 < R) {
    auto load_l = [&](int tj, bf16x8* bl) {
      const int j = tj * 64 + ch * 32 + l32;
      const bf16* lrow_p = lm + ((size_t)bg * NB + min(j, NB - 1)) * D;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        bl[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lrow_p + 16 * st + 8 * half));
        if (j >= NB) {
#pragma unroll
          for (int e = 0; e < 8; ++e) bl[st][e] = f2bf(0.0f);
        }
      }
    };
    // the wave's rows take every candidate of an interior tile and keep K = topk < n
    const bool rows_full = topk > 0 && row0 >= topk + n_local + n_sink && row0 + 31 < R;
    const uint32_t below = (1u << l32) - 1u;
    // column tile tj from the landmark fragments in cur, the next tile's loading into nxt;
    // false past the wave's last tile
    auto tile = [&](int tj, bf16x8* cur, bf16x8* nxt) -> bool {
      const int col0 = tj * 64 + ch * 32;
      if (tj > ti || col0 > last_row || col0 >= NB) return false;
      const int j = col0 + l32;
      if (tj + 1 <= ti) load_l(tj + 1, nxt);
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        acc = mfma32(hi[st], cur[st], acc);
        acc = mfma32(mid[st], cur[st], acc);
        acc = mfma32(lo[st], cur[st], acc);
      }
      uint32_t pbits = 0u;                     // bit i: append acc[i]
      if (rows_full && col0 >= n_sink && col0 + 31 <= row0 - n_local) {
#pragma unroll
        for (int i = 0; i < 16; ++i) pbits |= acc[i] > tau[i] ? (1u << i) : 0u;
      } else {                                 // tiles holding forced entries or row ends
#pragma unroll 1
        for (int i = 0; i < 16; ++i) {
          const int rr = row0 + 8 * (i / 4) + 4 * half + (i % 4);
          if (rr >= R || j > rr || j >= NB) continue;
          const float sv = acc[i];
          const int n_sink_eff = min(n_sink, rr + 1);
          const int n = max(0, rr - n_local - n_sink + 1);
          const int K = min(topk, n);
          const int loc_beg = max(n_sink, rr - n_local + 1);
          int opos = -1;
          if (j < n_sink_eff) opos = j;
          else if (j >= loc_beg) opos = n_sink_eff + K + (j - loc_beg);
          else if (K == n) opos = n_sink_eff + (j - n_sink);
          else if (K > 0 && sv > tau[i]) pbits |= 1u << i;
          if (opos >= 0) {
            oidx[(size_t)rr * NA + opos] = j;
            osc[(size_t)rr * NA + opos] = sv;
          }
        }
      }
      if (__any(pbits != 0u)) {
        uint32_t cutm = 0u;                    // lists (bit i) that the next tile could overflow
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool pi = (pbits >> i) & 1u;
          const uint32_t m = (uint32_t)(__ballot(pi) >> (32 * half));
          if (__any(m != 0u)) {
            int* cp = &lcnt[lrow(i)][ch];
            const int c0 = *cp;
            if (pi) {
              const int slot = ch * CAP + c0 + __popc(m & below);
              ls[lrow(i)][slot] = acc[i];
              lj[lrow(i)][slot] = (uint16_t)j;
            }
            const int c1 = c0 + __popc(m);
            if (l32 == 0) *cp = c1;
            cutm |= (c1 > CAP - 32) ? (1u << i) : 0u;
          }
        }
        uint32_t cuts = (uint32_t)(__builtin_amdgcn_readlane((int)cutm, 0) |
                                   __builtin_amdgcn_readlane((int)cutm, 32));
        if (cuts != 0u) {
#pragma unroll 1
          for (; cuts != 0u; cuts &= cuts - 1u) {
            const int i = __builtin_ctz(cuts);
            const int lr = rh * 32 + 8 * (i / 4) + 4 * half + (i % 4);
            const int rr = ti * 64 + lr;
            const int K = max(1, min(topk, max(0, rr - n_local - n_sink + 1)));
            const int c1 = lcnt[lr][ch];
            const uint32_t t = cut_list(&ls[lr][ch * CAP], &lj[lr][ch * CAP], c1, K, l32);
            if (l32 == 0 && c1 > K) {
              lcnt[lr][ch] = K;
              ltau[lr][ch] = key_float(t);
            }
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) tau[i] = ltau[lrow(i)][ch];
        }
      }
      return true;
    };
    bf16x8 bl[D / 16], bn[D / 16];
    load_l(0, bl);
    for (int tj = 0;; tj += 2) {
      if (!tile(tj, bl, bn)) break;
      if (!tile(tj + 1, bn, bl)) break;
    }
  }
  __syncthreads();

  // per row (one half-wave each): merge the two lists in block order, cut to K, write the
  // chosen entries and the padding
  const int hw = w * 2 + half;
  for (int r = hw; r < 64; r += 8) {
    const int rr = ti * 64 + r;
    if (rr >= R) break;
    const int n_sink_eff = min(n_sink, rr + 1);
    const int n = max(0, rr - n_local - n_sink + 1);
    const int K = min(topk, n);
    const int loc_beg = max(n_sink, rr - n_local + 1);
    const int n_loc = max(0, rr - loc_beg + 1);
    for (int p = n_sink_eff + K + n_loc + l32; p < NA; p += 32) {
      oidx[(size_t)rr * NA + p] = -1;
      osc[(size_t)rr * NA + p] = 0.0f;
    }
    if (K == 0 || K == n) continue;
    const int a = lcnt[r][0], b = lcnt[r][1];
    // list h holds blocks 64t + 32h + [0, 32) of tiles t in ascending order: an entry of list 0
    // from tile t follows the entries of list 1 from tiles < t, one of list 1 those of list 0
    // from tiles <= t
    float v[4];
    int jv[4], dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int h = u / 2;                      // u = 0, 1: list 0; 2, 3: list 1
      const int p = (u % 2) * 32 + l32;
      const int cn = h == 0 ? a : b, co = h == 0 ? b : a;
      dst[u] = -1;
      if (p < cn) {
        v[u] = ls[r][h * CAP + p];
        jv[u] = lj[r][h * CAP + p];
        const int t = jv[u] / 64;
        // entries of the other list with tile < t (list 0 asking) or <= t (list 1 asking)
        int lo_i = 0, hi_i = co;
        while (lo_i < hi_i) {
          const int mid_i = (lo_i + hi_i) / 2;
          const int to = lj[r][(1 - h) * CAP + mid_i] / 64;
          if (h == 0 ? to < t : to <= t) lo_i = mid_i + 1;
          else hi_i = mid_i;
        }
        dst[u] = p + lo_i;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (dst[u] >= 0) {
        ls[r][dst[u]] = v[u];
        lj[r][dst[u]] = (uint16_t)jv[u];
      }
    cut_list(&ls[r][0], &lj[r][0], a + b, K, l32);
    if (l32 < K) {
      oidx[(size_t)rr * NA + n_sink_eff + l32] = lj[r][l32];
      osc[(size_t)rr * NA + n_sink_eff + l32] = ls[r][l32];
    }
  }
}

bool select_fused_ok(const Shape& s) {
  return !s.decode && s.bf16 && s.topk <= kFusedMaxK && s.NB <= 65536 && s.R == s.NB;
}
// bsa_select_topk takes the one-pass kernel where it wins: rows of more than 4096 blocks (at 2048
// blocks a tile row is too little work per workgroup and the two-kernel path is faster)
bool select_fused(const Shape& s) { return select_fused_ok(s) && s.NB > 4096; }

hipError_t launch_select_fused(const Shape& s, const void* q, const void* lm, int32_t* idx,
                               float* sc, hipStream_t st) {
  const dim3 grid((s.R + 63) / 64, s.B * s.Hkv);
#define BSA_SF(D_)                                                                               \
  hipLaunchKernelGGL(select_fused_kernel<D_>, grid, dim3(256), 0, st, (const bf16*)q,           \
                     (const bf16*)lm, idx, sc, s.Hq, s.Hkv, s.G, s.Tq, s.R, s.NB, s.topk,       \
                     s.n_sink, s.n_local, s.NA)
  if (s.D == 128) BSA_SF(128);
  else BSA_SF(64);
#undef BSA_SF
  return hipGetLastError();
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
