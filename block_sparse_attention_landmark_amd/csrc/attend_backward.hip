// Backward pass of PLAIN / SAS block-sparse prefill attention (bf16 inputs, float32 arithmetic).
//
// For the attended sets of a forward pass (SAS page, summary paragraphs 2-3: the selector is
// trained end to end through the gates inside the softmax), per query row t and attended key u:
//   x = scale q.k_u + g_j(u),  P = exp(x - lse),  dP = do.v_u,  dx = P (dP - do.o),
//   dq = scale sum_u dx k_u,  dk_u = scale sum_t dx q_t,  dv_u = sum_t P do_t,
//   dg_j = sum over the rows of query block c (all heads of the group) and keys of block j of dx,
//   g_j = log sigmoid(S_j - S_c): d S_j = dg_j sigmoid(S_c - S_j), d S_c -= the same (j != c).
//
// Kernels, in launch order:
//   bwd_delta_kernel        Delta = do . o per query row (float32);
//   bwd_count/scan/fill     the inverse of the attended sets: for every key block j of every
//                           (sequence, kv group) the entries (c, pos) that attend it, grouped by
//                           j, sorted (bwd_sort_kernel) so sums are deterministic, and cut into
//                           work items of kBwdChunk entries;
//   bwd_dq_kernel           one workgroup per (query block, kv group, head chunk): for each
//                           attended block, S^T = K Q^T, dP^T = V dO^T (MFMA), dx, then
//                           dQ^T += K^T dx^T (MFMA, K read transposed); sums dx per block into dg
//                           and stores each entry's gate;
//   bwd_dkdv_kernel         one workgroup per work item (key block j, up to kBwdChunk entries):
//                           K_j and V_j stay in registers; for each entry and head it copies Q and
//                           dO of the query block into LDS a few steps ahead, forms S = Q K^T,
//                           dP = dO V^T, dx, and accumulates dV^T += dO^T P and dK^T += Q^T dx
//                           (MFMA) for its keys; a key block's only work item writes dk, dv;
//   bwd_reduce_kernel       otherwise sums the block's work-item partials in order and writes;
//   bwd_dsc_kernel          the selector-score gradient of each attended-set row (SAS).
// The MFMA layouts are those of the forward kernels (32x32x16 bf16; see attend_prefill.hip).
#include <math.h>

#include <algorithm>

#include "attend_common.hpp"
#include "bsa_internal.hpp"

namespace bsa {

constexpr int kBwdChunk = 64;        // attended entries per dK/dV work item
constexpr int kBwdSortCap = 4096;    // longer entry lists of one key block are left unsorted

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------------------------
// workspace
// ---------------------------------------------------------------------------------------------
struct BwdWs {
  float* delta;   // [B, Hq, T]
  float* dg;      // [B, Hkv, R, NA]
  float* gates;   // [B, Hkv, R, NA] gate of each entry, log2 units
  int* cnt_off;   // [B*Hkv, NB + 1]: counts, then exclusive offsets
  int* cursor;    // [B*Hkv, NB]
  int* chunk_off; // [B*Hkv, NB + 1]
  int* work;      // [B*Hkv, max_work]: j | chunk << 16
  int* n_work;    // [B*Hkv]
  int* list;      // [B*Hkv, R * NA]: c * NA + pos, grouped by key block
  float* part;    // [B*Hkv, max_work, 2, 64, D]: dK then dV partial tiles (unscaled)
  float* hstat;   // HiLS: 3 x [B, Hq, R, NA, 64] row statistics (softmax bias, dw, dr)
  size_t hs_n;    // elements of one of them
  float* partL;   // HiLS: [B*Hkv, max_work, D] landmark-gradient partials (unscaled)
};

static int bwd_max_work(const Shape& s) {
  return (int)(((int64_t)s.R * s.NA + kBwdChunk - 1) / kBwdChunk) + s.NB;
}

static size_t bwd_layout(const Shape& s, char* base, BwdWs* w) {
  const size_t BG = (size_t)s.B * s.Hkv;
  const size_t rowsel = BG * s.R * s.NA;
  const size_t mw = (size_t)bwd_max_work(s);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += al256(bytes);
    return p;
  };
  BwdWs x;
  x.delta = (float*)take((size_t)s.B * s.Hq * s.Tq * 4);
  x.dg = (float*)take(rowsel * 4);
  x.gates = (float*)take(rowsel * 4);
  x.cnt_off = (int*)take(BG * (s.NB + 1) * 4);
  x.cursor = (int*)take(BG * s.NB * 4);
  x.chunk_off = (int*)take(BG * (s.NB + 1) * 4);
  x.work = (int*)take(BG * mw * 4);
  x.n_work = (int*)take(BG * 4);
  x.list = (int*)take(rowsel * 4);
  x.part = (float*)take(BG * mw * 2 * kBlock * s.D * 4);
  x.hs_n = s.mode == 2 ? (size_t)s.B * s.Hq * s.R * s.NA * kBlock : 0;
  x.hstat = (float*)take(3 * x.hs_n * 4);
  x.partL = (float*)take(s.mode == 2 ? BG * mw * s.D * 4 : 0);
  if (w) *w = x;
  return off;
}

size_t backward_ws_bytes(const Shape& s) { return bwd_layout(s, nullptr, nullptr); }

// ---------------------------------------------------------------------------------------------
// Delta = do . o, D / 8 lanes per row
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const bf16* __restrict__ out,
                                                        const bf16* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t rows) {
  constexpr int LPR = D / 8;
  constexpr int RPW = kWave / LPR;
  const int64_t r = ((int64_t)blockIdx.x * 4 + threadIdx.x / kWave) * RPW + (threadIdx.x % kWave) / LPR;
  const int part = threadIdx.x % LPR;
  float s = 0.0f;
  if (r < rows) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(out + r * D + part * 8));
    const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dout + r * D + part * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(bf2f(a[e]), bf2f(b[e]), s);
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (r < rows && part == 0) delta[r] = s;
}

// ---------------------------------------------------------------------------------------------
// inverse of the attended sets
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_fill_zero_kernel(int* __restrict__ p, int64_t n,
                                                            float* __restrict__ f, int64_t nf) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nf; i += (int64_t)gridDim.x * 256) f[i] = 0.0f;
}

__global__ __launch_bounds__(256) void bwd_count_kernel(const int32_t* __restrict__ idx,
                                                        int* __restrict__ cnt, int R, int NA,
                                                        int NB, int64_t n_entries) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_entries) return;
  const int64_t row = e / NA;
  const int bg = (int)(row / R), c = (int)(row % R);
  const int j = idx[e];
  if (j >= 0 && j <= c && j < NB) atomicAdd(&cnt[(int64_t)bg * (NB + 1) + j], 1);
}

// exclusive scan over a 1024-thread workgroup
__device__ __forceinline__ int bwd_block_scan(int x, int* sbuf, int* total) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int incl = x;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) sbuf[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < 16; ++i) {
    const int v = sbuf[i];
    base += (i < w) ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

// one workgroup of 1024 threads per (sequence, kv group)
__global__ __launch_bounds__(1024) void bwd_scan_kernel(int* __restrict__ cnt_off,
                                                        int* __restrict__ cursor,
                                                        int* __restrict__ chunk_off,
                                                        int* __restrict__ work,
                                                        int* __restrict__ n_work, int NB,
                                                        int max_work) {
  __shared__ int sbuf[16];
  const int bg = blockIdx.x;
  int* cnt = cnt_off + (int64_t)bg * (NB + 1);
  int* cur = cursor + (int64_t)bg * NB;
  int* coff = chunk_off + (int64_t)bg * (NB + 1);
  int* wl = work + (int64_t)bg * max_work;
  const int per = (NB + 1023) / 1024;
  const int beg = min(NB, (int)threadIdx.x * per), end = min(NB, beg + per);
  int s_cnt = 0, s_ch = 0;
  for (int j = beg; j < end; ++j) {
    s_cnt += cnt[j];
    s_ch += (cnt[j] + kBwdChunk - 1) / kBwdChunk;
  }
  int tot_cnt, tot_ch;
  int o_cnt = bwd_block_scan(s_cnt, sbuf, &tot_cnt);
  int o_ch = bwd_block_scan(s_ch, sbuf, &tot_ch);
  for (int j = beg; j < end; ++j) {
    const int n = cnt[j];
    const int nch = (n + kBwdChunk - 1) / kBwdChunk;
    cnt[j] = o_cnt;
    cur[j] = o_cnt;
    coff[j] = o_ch;
    for (int ch = 0; ch < nch; ++ch) wl[o_ch + ch] = j | (ch << 16);
    o_cnt += n;
    o_ch += nch;
  }
  if (threadIdx.x == 0) {
    cnt[NB] = tot_cnt;
    coff[NB] = tot_ch;
    n_work[bg] = tot_ch;
  }
}

__global__ __launch_bounds__(256) void bwd_fill_kernel(const int32_t* __restrict__ idx,
                                                       int* __restrict__ cursor,
                                                       int* __restrict__ list, int R, int NA,
                                                       int NB, int64_t n_entries) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_entries) return;
  const int64_t row = e / NA;
  const int bg = (int)(row / R), c = (int)(row % R), pos = (int)(e % NA);
  const int j = idx[e];
  if (j >= 0 && j <= c && j < NB) {
    const int slot = atomicAdd(&cursor[(int64_t)bg * NB + j], 1);
    list[(int64_t)bg * R * NA + slot] = c * NA + pos;
  }
}

// one workgroup per (key block, sequence x kv group): bitonic sort of the block's entries
__global__ __launch_bounds__(256) void bwd_sort_kernel(const int* __restrict__ cnt_off,
                                                       int* __restrict__ list, int R, int NA,
                                                       int NB) {
  __shared__ int buf[kBwdSortCap];
  const int j = blockIdx.x, bg = blockIdx.y;
  const int off = cnt_off[(int64_t)bg * (NB + 1) + j];
  const int n = cnt_off[(int64_t)bg * (NB + 1) + j + 1] - off;
  if (n <= 1 || n > kBwdSortCap) return;
  int* seg = list + (int64_t)bg * R * NA + off;
  int m = 1;
  while (m < n) m <<= 1;
  for (int i = threadIdx.x; i < m; i += 256) buf[i] = i < n ? seg[i] : 0x7fffffff;
  __syncthreads();
  for (int k = 2; k <= m; k <<= 1)
    for (int s = k >> 1; s > 0; s >>= 1) {
      for (int i = threadIdx.x; i < m; i += 256) {
        const int p = i ^ s;
        if (p > i) {
          const bool up = (i & k) == 0;
          const int a = buf[i], b2 = buf[p];
          if ((a > b2) == up) {
            buf[i] = b2;
            buf[p] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < n; i += 256) seg[i] = buf[i];
}

// ---------------------------------------------------------------------------------------------
// dQ (and the per-entry gate gradient sums)
// ---------------------------------------------------------------------------------------------
template <int D, int MODE, int HPW>
__global__ __launch_bounds__(HPW * 128) void bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ idx, const float* __restrict__ sc, const bf16* __restrict__ lm,
    bf16* __restrict__ dq, float* __restrict__ dg, float* __restrict__ gates_out,
    float* __restrict__ hstat, size_t hs_n, int Hq, int Hkv, int G, int T, int NQB, int NA,
    int n_hc, float scale_log2, float scale) {
  constexpr int NT = HPW * 128;
  constexpr int NWAVE = HPW * 2;
  constexpr int KP = D + 8;            // V and landmark tile row pitch (elements)
  // K tile row pitch: K is read both as rows (S) and transposed (dQ).  At D = 128, rows 12 banks
  // apart keep the row reads free of bank conflicts and the transposed reads of 32 lanes at most
  // two to a bank (rows 4 banks apart, as D + 8 gives, put up to four on one bank)
  constexpr int KPK = D == 128 ? D + 24 : D + 8;
  constexpr int C8 = D / 8;
  constexpr int CPT = kBlock * C8 / NT;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][kBlock * KPK];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][kBlock * KP];
  // HiLS: landmark rows of the attended chunks, and per (wave, entry, row) the retrieval weight
  // (overwritten by the retrieval-score gradient after the entry loop); dw = dout . o_j of each
  // (row, entry) is kept in the row statistics for the key side and read back from there
  __shared__ __attribute__((aligned(16))) bf16 Lb[MODE == 2 ? kBlock * KP : 8];
  __shared__ float wbuf[MODE == 2 ? NWAVE * 64 * 32 : 1];
  float g_acc = 0.0f;                  // HiLS: sum_j w_j dw_j = dout . o, accumulated exactly

  const int c = NQB - 1 - (int)blockIdx.x;   // heavy (late) query blocks first
  const int g = blockIdx.y / n_hc, hc = blockIdx.y % n_hc;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int half = lane / 32, l32 = lane % 32;
  const int h = g * G + hc * HPW + w / 2;
  const int tq = c * kBlock + (w % 2) * 32 + l32;
  const bool row_ok = tq < T;
  const size_t qrow_off = ((size_t)(b * Hq + h) * T + min(tq, T - 1)) * D;

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 a = *reinterpret_cast<const u32x4*>(q + qrow_off + 16 * s + 8 * half);
    u32x4 bb = *reinterpret_cast<const u32x4*>(dout + qrow_off + 16 * s + 8 * half);
    if (!row_ok) a = bb = u32x4{0u, 0u, 0u, 0u};
    qf[s] = __builtin_bit_cast(bf16x8, a);
    df[s] = __builtin_bit_cast(bf16x8, bb);
  }
  const size_t rrow = (size_t)(b * Hq + h) * T + min(tq, T - 1);
  const float lse2 = (MODE != 2 && row_ok) ? lse[rrow] * kLog2e : 0.0f;
  const float dlt = row_ok ? delta[rrow] : 0.0f;

  const size_t kvbase = (size_t)(b * Hkv + g) * T * D;
  const size_t rowsel = ((size_t)(b * Hkv + g) * NQB + c) * NA;
  const int32_t* irow = idx + rowsel;
  const int nval = count_valid(irow, NA);
  float s_ref = 0.0f;
  if (MODE == 1 && nval > 0) s_ref = sc[rowsel + nval - 1];
  auto gate_of = [&](int a, int j) {
    if (MODE != 1 || j == c) return 0.0f;
    return log_sigmoid(sc[rowsel + a] - s_ref) * kLog2e;
  };
  if (MODE != 2 && hc == 0 && w == 0)
    for (int a = lane; a < nval; a += kWave) {
      const int j = irow[a];
      gates_out[rowsel + a] = gate_of(a, j);
    }
  // HiLS: retrieval logits (log2 units) of the entries e0 .. e0+63 for this wave's 32 rows
  // (-inf past nval), R^T = L Q^T on MFMA as in the forward, and their weights
  // softmax_j(scale q . L_j) over every attended chunk (max and 1 / sum carried over groups of
  // 64) into this wave's table.  The landmark rows of the group held in Lb are read from LDS
  // (from_lds); those of other groups straight from memory as A fragments.
  float w_max = -INFINITY, w_inv = 0.0f;
  auto hils_logits = [&](int e0, f32x16* rt, bool from_lds) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int e = e0 + kt * 32 + l32;
      const int jr = e < nval ? irow[e] : -1;
      const bool ok = jr >= 0 && jr <= c;
      const bf16* lrow = lm + ((size_t)(b * Hkv + g) * NQB + (ok ? jr : 0)) * D + 8 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i) rt[kt][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        bf16x8 a;
        if (from_lds) {
          a = *reinterpret_cast<const bf16x8*>(&Lb[(kt * 32 + l32) * KP + 16 * s + 8 * half]);
        } else {
          u32x4 raw = *reinterpret_cast<const u32x4*>(lrow + 16 * s);
          if (!ok) raw = u32x4{0u, 0u, 0u, 0u};
          a = __builtin_bit_cast(bf16x8, raw);
        }
        rt[kt] = mfma32(a, qf[s], rt[kt]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = e0 + kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        rt[kt][i] = slot < nval ? rt[kt][i] * scale_log2 : -INFINITY;
      }
    }
  };
  auto hils_weights = [&](const f32x16* rt) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        wbuf[(w * 64 + slot) * 32 + l32] = fast_exp2(rt[kt][i] - w_max) * w_inv;
      }
  };
  // HiLS: the landmark rows of the entries e0 .. e0+63 into Lb (zero rows past nval)
  auto stage_landmarks = [&](int e0) {
    for (int ci = tid; ci < kBlock * C8; ci += NT) {
      const int row = ci / C8, c8 = ci % C8;
      const int e = e0 + row;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      const int jr = e < nval ? irow[e] : -1;
      if (jr >= 0 && jr <= c)
        val = *reinterpret_cast<const u32x4*>(lm + ((size_t)(b * Hkv + g) * NQB + jr) * D + c8 * 8);
      *reinterpret_cast<u32x4*>(&Lb[row * KP + c8 * 8]) = val;
    }
  };
  const int ngr = (nval + 63) / 64;              // HiLS: groups of 64 entries
  if constexpr (MODE == 2) {
    stage_landmarks(0);
    __syncthreads();
    f32x16 rt[2];
    float den = 0.0f;
    for (int gi = 0; gi < ngr; ++gi) {
      hils_logits(gi * 64, rt, gi == 0);
      float mloc = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, rt[kt][i]);
      const float m_new = fmaxf(w_max, wave_max_xor32(mloc));
      float dsum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) dsum += fast_exp2(rt[kt][i] - m_new);
      dsum = wave_sum_xor32(dsum);
      den = gi == 0 ? dsum : den * fast_exp2(w_max - m_new) + dsum;
      w_max = m_new;
    }
    if (ngr > 0) {
      w_inv = 1.0f / den;
      if (ngr > 1) hils_logits(0, rt, true);
      hils_weights(rt);
    }
  }

  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int a) {
    const int j = irow[a];
    const bool ok = j >= 0 && j <= c;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + i * NT;
      const int row = ci / C8, c8 = ci % C8;
      const int tok = j * kBlock + row;
      kreg[i] = vreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (ok && tok < T) {
        kreg[i] = *reinterpret_cast<const u32x4*>(k + kvbase + (size_t)tok * D + c8 * 8);
        vreg[i] = *reinterpret_cast<const u32x4*>(v + kvbase + (size_t)tok * D + c8 * 8);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + i * NT;
      const int row = ci / C8, c8 = ci % C8;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KPK + c8 * 8]) = kreg[i];
      *reinterpret_cast<u32x4*>(&Vs[buf][row * KP + c8 * 8]) = vreg[i];
    }
  };

  f32x16 dqa[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[dt][i] = 0.0f;
  const int vrow = (lane % 16) / 4;
  const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);

  if (nval > 0) load_tile(0);
  if (nval > 0) store_tile(0);
  if (nval > 1) load_tile(1);
  __syncthreads();
  for (int a = 0; a < nval; ++a) {
    const int buf = a & 1;
    const int j = irow[a];
    if constexpr (MODE == 2) {
      if (a > 0 && a % 64 == 0) {               // the weights of the next 64 entries
        f32x16 rt[2];
        hils_logits(a, rt, false);
        hils_weights(rt);
      }
    }
    if (j >= 0 && j <= c) {
      // a block before the query block, all of whose rows are in the sequence, has no masked
      // key; for the others the masked scores are set to -inf (exp2 then gives 0)
      const bool full = j < c && (c + 1) * kBlock <= T;
      const bf16* Kb = Ks[buf];
      const bf16* Vb = Vs[buf];
      f32x16 st[2], dp[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) st[kt][i] = dp[kt][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const int col = 16 * s + 8 * half;
          const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(&Kb[(kt * 32 + l32) * KPK + col]);
          const bf16x8 vfr = *reinterpret_cast<const bf16x8*>(&Vb[(kt * 32 + l32) * KP + col]);
          st[kt] = mfma32(kfr, qf[s], st[kt]);
          dp[kt] = mfma32(vfr, df[s], dp[kt]);
        }
      }
      if (!full) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j * kBlock + kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
            if (!(row_ok && key <= tq)) st[kt][i] = -INFINITY;
          }
      }
      if constexpr (MODE == 2) {
        // HiLS: softmax of the row over this chunk's visible keys alone (P), dw = dout . o_j,
        // dx = w_j P (dP - dw); dr_j = w_j (dw_j - sum_i w_i dw_i) is formed after the loop
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kt][i]);
        mx = wave_max_xor32(mx);
        const float mxs = mx == -INFINITY ? 0.0f : mx * scale_log2;
        float l = 0.0f, dwp = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(fmaf(st[kt][i], scale_log2, -mxs));
            st[kt][i] = p;
            l += p;
            dwp = fmaf(p, dp[kt][i], dwp);
          }
        l = wave_sum_xor32(l);
        dwp = wave_sum_xor32(dwp);
        const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
        const float dwv = dwp * inv_l;
        const float wj = wbuf[(w * 64 + a % 64) * 32 + l32];
        g_acc = fmaf(wj, dwv, g_acc);
        const float coef = wj * inv_l;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) st[kt][i] = coef * st[kt][i] * (dp[kt][i] - dwv);
        if (half == 0) {
          // row statistics for the key side: w_j P = exp2(scale_log2 s - bias)
          const size_t hi = (((size_t)(b * Hq + h) * NQB + c) * NA + a) * kBlock + (w % 2) * 32 + l32;
          const bool live = row_ok && l > 0.0f && wj > 0.0f;
          hstat[hi] = live ? mxs + log2f(l) - log2f(wj) : 0.0f;
          hstat[hs_n + hi] = live ? dwv : 0.0f;
        }
      } else {
        const float gb = gate_of(a, j) - lse2;
        float dgs = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(fmaf(st[kt][i], scale_log2, gb));
            const float x = p * (dp[kt][i] - dlt);
            st[kt][i] = x;
            dgs += x;
          }
        // gate gradient of this entry: the sum over the wave's rows and keys
        if constexpr (MODE == 1) {
          const float tot = wave_sum64(dgs);
          if (lane == 0) atomicAdd(&dg[rowsel + a], tot);
        }
      }
      // dQ^T += K^T dx^T: the K tile read transposed, dx^T from the score registers
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 xb;
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[e] = f2bf(st[ks / 2][8 * (ks % 2) + e]);
        const bf16* k0 = Kb + (16 * ks + 4 * half + vrow) * KPK + vcol;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const i16x4 x0 = lds_read_tr16(k0 + dt * 32);
          const i16x4 x1 = lds_read_tr16(k0 + 8 * KPK + dt * 32);
          const bf16x8 ak = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          dqa[dt] = mfma32(ak, xb, dqa[dt]);
        }
      }
    }
    if (a + 1 < nval) store_tile(buf ^ 1);
    if (a + 2 < nval) load_tile(a + 2);
    __syncthreads();
  }
  if constexpr (MODE == 2) {
    // per group of 64 entries: the retrieval-score gradients dr_j = w_j (dw_j - sum_i w_i dw_i),
    // kept for the key side, then dQ^T += L^T dR^T with the group's landmark rows in LDS
    for (int gi = 0; gi < ngr; ++gi) {
      const int e0 = gi * 64;
      if (ngr > 1) {                             // one group: its weights are still in the table
        f32x16 rt[2];
        hils_logits(e0, rt, false);
        hils_weights(rt);
      }
      if (half == 0)
        for (int a = e0; a < min(nval, e0 + 64); ++a) {
          const int sl = (w * 64 + a - e0) * 32 + l32;
          const size_t hi = (((size_t)(b * Hq + h) * NQB + c) * NA + a) * kBlock + (w % 2) * 32 + l32;
          // dw of this row and entry as stored for the key side (0 where the weight is 0, and
          // there dr is 0 either way)
          const float dwj = hstat[hs_n + hi];
          const float wj = wbuf[sl];
          const float drv = row_ok ? wj * (dwj - g_acc) : 0.0f;
          hstat[2 * hs_n + hi] = drv;
          wbuf[sl] = drv;
        }
      if (gi > 0) {                              // group 0's rows are still in Lb
        __syncthreads();                         // the previous group's rows have been read
        stage_landmarks(e0);
        __syncthreads();
      }
      // the transposed landmark reads put chunks 16ks + 4half + {0..3} and 16ks + 8 + 4half +
      // {0..3} in a lane's k slots, and the retrieval-score gradients are taken in that order
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 rb;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          rb[e] = f2bf(wbuf[(w * 64 + 16 * ks + 4 * half + (e % 4) + 8 * (e / 4)) * 32 + l32]);
        const bf16* l0 = Lb + (16 * ks + 4 * half + vrow) * KP + vcol;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const i16x4 x0 = lds_read_tr16(l0 + dt * 32);
          const i16x4 x1 = lds_read_tr16(l0 + 8 * KP + dt * 32);
          const bf16x8 al = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          dqa[dt] = mfma32(al, rb, dqa[dt]);
        }
      }
    }
  }
  if (row_ok) {
    bf16* orow = dq + ((size_t)(b * Hq + h) * T + tq) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = f2bf(dqa[dt][4 * i4 + e] * scale);
        *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * i4 + 4 * half) = ov;
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV of one work item: key block j, entries [e0, e1) of its list, all heads of the group
// ---------------------------------------------------------------------------------------------
// Four waves; wave w owns keys kh*32..+32 (kh = w % 2) and query rows th*32..+32 (th = w / 2) of
// every step, so S and dP are formed once.  K_j and V_j stay in registers as MFMA B fragments for
// the whole item.  Step s = (entry s / G, head s % G) needs Q and dO of that query block and head
// (64 x D each) plus lse and Delta of its 64 rows; they are copied from global memory straight
// into LDS (dma_lds) kBwdAhead steps ahead, in kBwdStages rotating stages, one barrier per step.
// No other vector memory instruction is issued inside the step loop (the per-entry block and gate
// are staged in LDS first), so the copy counter waits below count exactly those copies.
// Tiles are stored with the 16-byte chunks of row r XOR-swizzled by bwd_swz(r): conflict-free
// both for row reads (the A operands of S and dP) and for transposed reads (dO^T, Q^T).
constexpr int kBwdStages = 4;
constexpr int kBwdAhead = kBwdStages - 1;

template <int D>
__device__ __forceinline__ int bwd_swz(int r) {
  if constexpr (D == 128) return (4 * (r % 4)) ^ ((r / 4) % 4);
  return 4 * ((r / 2) % 2) + ((r / 4) % 4);
}
// element offset of (row, col) in a swizzled 64 x D tile
template <int D>
__device__ __forceinline__ int bwd_tile_off(int row, int col) {
  return row * D + 8 * ((col >> 3) ^ bwd_swz<D>(row)) + (col & 7);
}

__device__ __forceinline__ void bwd_wait_copies(int left) {
  // s_waitcnt with expcnt and lgkmcnt at their maxima and vmcnt = left (split over two fields)
#define BSA_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
  switch (left) {
    case 0: BSA_VM(0); break;
    case 5: BSA_VM(5); break;
    case 9: BSA_VM(9); break;
    case 10: BSA_VM(10); break;
    case 18: BSA_VM(18); break;
    default: BSA_VM(0); break;
  }
#undef BSA_VM
}

// (at D = 64 a wave's registers fit two workgroups per CU; at D = 128 one wave per SIMD holds
// about 420)
template <int D, int MODE>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ gates, const int* __restrict__ cnt_off,
    const int* __restrict__ chunk_off, const int* __restrict__ list, const int* __restrict__ work,
    const int* __restrict__ n_work, float* __restrict__ part, bf16* __restrict__ dk,
    bf16* __restrict__ dv, const float* __restrict__ hstat, size_t hs_n, float* __restrict__ partL,
    float* __restrict__ dlm, int Hq, int Hkv, int G, int T, int NQB, int NB, int NA, int max_work,
    float scale_log2, float scale) {
  constexpr int C = D / 8;                       // 16-byte chunks per row
  constexpr int TILE_B = kBlock * D * 2;         // bytes of one 64 x D bf16 tile
  constexpr int CPW = TILE_B / 16 / 256;         // copies of one tile per wave and step
  constexpr int NPS = 2 * CPW + 1;               // copy instructions per wave and step
  constexpr int STAGE_B = 2 * TILE_B + 4 * kBlock * 4;
  constexpr int DT = D / 32;                     // 32-column d tiles
  static_assert(NPS == 5 || NPS == 9, "copy counts must match bwd_wait_copies");
  __shared__ __attribute__((aligned(16))) char smem[kBwdStages * STAGE_B];
  __shared__ int Ec[kBwdChunk];
  __shared__ float Eg[kBwdChunk];
  __shared__ int Ep[kBwdChunk];                  // HiLS: the entry's position in its row
  __shared__ float Lred[MODE == 2 ? 2 * D : 1];

  const int g = blockIdx.y, b = blockIdx.z;
  const int bg = b * Hkv + g;
  const int wi = blockIdx.x;
  if (wi >= n_work[bg]) return;                  // whole workgroup, before any barrier
  const int item = work[(size_t)bg * max_work + wi];
  const int j = item & 0xffff, ch = item >> 16;
  const int* co = cnt_off + (size_t)bg * (NB + 1);
  const int e0 = co[j] + ch * kBwdChunk;
  const int ne = min(co[j + 1] - e0, kBwdChunk);
  const int nch = chunk_off[(size_t)bg * (NB + 1) + j + 1] - chunk_off[(size_t)bg * (NB + 1) + j];
  const int* lst = list + (size_t)bg * NQB * NA;

  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int half = lane / 32, l32 = lane % 32;
  const int kh = w % 2, th = w / 2;
  const int ku = j * kBlock + kh * 32 + l32;     // this lane's key (the n index of S)
  const size_t kvbase = (size_t)bg * T * D;

  if (tid < ne) {
    const int ent = lst[e0 + tid];
    const int c = ent / NA;
    Ec[tid] = c;
    Ep[tid] = ent % NA;
    Eg[tid] = MODE == 1 ? gates[((size_t)bg * NQB + c) * NA + ent % NA] : 0.0f;
  }
  // K_j and V_j rows of this wave's keys as B fragments: B[k = d][n = key]
  bf16x8 kb[D / 16], vb[D / 16];
  {
    const int tok = min(ku, T - 1);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(k + kvbase + (size_t)tok * D + 16 * s + 8 * half));
      vb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(v + kvbase + (size_t)tok * D + 16 * s + 8 * half));
    }
    // keep these loads ahead of the first copy: the copy waits below count copies only
#pragma unroll
    for (int s = 0; s < D / 16; ++s) asm volatile("" : "+v"(kb[s]), "+v"(vb[s]));
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
  __syncthreads();

  const int nsteps = ne * G;
  const uint32_t smem_lds = lds_addr_of(smem);
  auto issue = [&](int st) {
    const int c = Ec[st / G];
    const int h = g * G + st % G;
    const int rmax = T - 1 - c * kBlock;         // last valid row of this query block
    const size_t row0 = (size_t)(b * Hq + h) * T + (size_t)c * kBlock;
    const char* qg = reinterpret_cast<const char*>(q + row0 * D);
    const char* og = reinterpret_cast<const char*>(dout + row0 * D);
    const uint32_t st_lds = smem_lds + (uint32_t)((st % kBwdStages) * STAGE_B);
    sync_copies_barrier();     // race-check build only (every wave issues every step's copies)
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int slot = (i * 4 + w) * kWave + lane;
      const int row = slot / C, pc = slot % C;
      const uint32_t voff = (uint32_t)(min(row, rmax) * (D * 2) + ((pc ^ bwd_swz<D>(row)) * 16));
      const uint32_t la = st_lds + (uint32_t)((i * 4 + w) * kWave * 16);
      dma_lds<16>(qg, voff, la);
      dma_lds<16>(og, voff, la + TILE_B);
    }
    if constexpr (MODE == 2) {
      // HiLS row statistics of this (query block, entry, head): softmax bias (wave 0), dw
      // (wave 1), retrieval-score gradient (wave 2); wave 3 fills an unused copy so that every
      // wave issues the same number of copies per step
      const size_t hrow = (((size_t)(b * Hq + h) * NQB + c) * NA + Ep[st / G]) * kBlock;
      const float* src = hstat + (size_t)(w % 3) * hs_n + hrow;
      dma_lds<4>(reinterpret_cast<const char*>(src), (uint32_t)(lane * 4),
                 st_lds + 2 * TILE_B + (uint32_t)(w * kBlock * 4));
    } else {
      // lse (waves 0, 2) and Delta (waves 1, 3); waves 2 and 3 fill a second, unused copy so
      // that every wave issues the same number of copies per step
      const float* src = (w % 2 == 0) ? lse : delta;
      dma_lds<4>(reinterpret_cast<const char*>(src + row0), (uint32_t)(min(lane, rmax) * 4),
                 st_lds + 2 * TILE_B + (uint32_t)(w * kBlock * 4));
    }
    sync_copies_barrier();
  };

  f32x16 dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[dt][i] = dva[dt][i] = 0.0f;
  float dla[DT];                                 // HiLS: dL for column dt*32 + l32, this lane's rows
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dla[dt] = 0.0f;

  const int vrow = (lane % 16) / 4;
  const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
  for (int s = 0; s < kBwdAhead; ++s)
    if (s < nsteps) issue(s);
  const int arow = th * 32 + l32;
  const int tb = th * 32 + 4 * half;
  // S = Q K^T and dP = dO V^T of step st for rows th*32..+32 and this wave's 32 keys, from its
  // stage; each accumulator sums its products in k-step order
  auto s_dp = [&](int st, f32x16& sa, f32x16& pa) {
    const char* stg = smem + (st % kBwdStages) * STAGE_B;
    const bf16* Qb = reinterpret_cast<const bf16*>(stg);
    const bf16* Ob = reinterpret_cast<const bf16*>(stg + TILE_B);
    bf16x8 qa[D / 16], oa[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int off = bwd_tile_off<D>(arow, 16 * s + 8 * half);
      qa[s] = *reinterpret_cast<const bf16x8*>(&Qb[off]);
      oa[s] = *reinterpret_cast<const bf16x8*>(&Ob[off]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sa[i] = pa[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) sa = mfma32(qa[s], kb[s], sa);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) pa = mfma32(oa[s], vb[s], pa);
  };
  // Software pipeline over the steps (one wave per SIMD, so nothing else fills the matrix
  // core): iteration st forms S and dP of step st + 1 -- products that need nothing of step
  // st -- while the vector work of step st (P, dx) runs, then step st's dV and dK products.
  // So stages st and st + 1 are read in iteration st, and the copies of step st + 1 must have
  // landed at its start; steps st + 2 and st + 3 may still be in flight.
  f32x16 sa, pa;
  if (nsteps > 0) {
    bwd_wait_copies(NPS * min(nsteps - 1, kBwdAhead - 1));   // step 0 has landed
    __syncthreads();
    s_dp(0, sa, pa);
  }
  for (int st = 0; st < nsteps; ++st) {
    if (st + 1 < nsteps)                        // step st + 1 has landed
      bwd_wait_copies(NPS * (min(nsteps - 1, st + kBwdAhead - 1) - (st + 1)));
    __syncthreads();                            // and every wave is done with stage st - 1
    if (st + kBwdAhead < nsteps) issue(st + kBwdAhead);
    const char* stg = smem + (st % kBwdStages) * STAGE_B;
    const bf16* Qb = reinterpret_cast<const bf16*>(stg);
    const bf16* Ob = reinterpret_cast<const bf16*>(stg + TILE_B);
    const float* Lb = reinterpret_cast<const float*>(stg + 2 * TILE_B);
    const float* Db = Lb + kBlock;
    const int c = Ec[st / G];
    const float gb = Eg[st / G];
    // a query block after the key block, all of whose rows are in the sequence, sees every key;
    // for the others the masked scores are set to -inf here (exp2 then gives 0)
    if (!(c > j && (c + 1) * kBlock <= T)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tq = c * kBlock + tb + 8 * (r / 4) + r % 4;
        if (!(tq < T && ku <= tq)) sa[r] = -INFINITY;
      }
    }
    // Step st + 1's stage: its Q and dO rows, the A operands of its S and dP products (in the
    // last step this reads a stage that holds no step; those products are discarded).
    const char* stn = smem + ((st + 1) % kBwdStages) * STAGE_B;
    const bf16* Qn = reinterpret_cast<const bf16*>(stn);
    const bf16* On = reinterpret_cast<const bf16*>(stn + TILE_B);
    bf16x8 qa[D / 16], oa[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int off = bwd_tile_off<D>(arow, 16 * s + 8 * half);
      qa[s] = *reinterpret_cast<const bf16x8*>(&Qn[off]);
      oa[s] = *reinterpret_cast<const bf16x8*>(&On[off]);
    }
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      l4[i4] = *reinterpret_cast<const f32x4*>(&Lb[tb + 8 * i4]);
      d4[i4] = *reinterpret_cast<const f32x4*>(&Db[tb + 8 * i4]);
    }
    // P and dx of step st in 16 / (D / 16) element chunks, each issued behind one S (then dP)
    // product of step st + 1: the products need nothing of step st, so the matrix core and the
    // vector unit work side by side.  Register i holds row t = th*32 + 8 (i / 4) + 4 half + i % 4.
    constexpr int PC = 16 / (D / 16);            // elements per chunk
    f32x16 sn, pn;
#pragma unroll
    for (int i = 0; i < 16; ++i) sn[i] = pn[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      sn = mfma32(qa[s], kb[s], sn);
#pragma unroll
      for (int r = s * PC; r < (s + 1) * PC; ++r) {
        const int i4 = r / 4, e = r % 4;
        const float bias = MODE == 2 ? -l4[i4][e] : gb - l4[i4][e] * kLog2e;
        sa[r] = fast_exp2(fmaf(sa[r], scale_log2, bias));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the transposed operands of step st's dV and dK products
    i16x4 tr[2][DT][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r0 = th * 32 + 16 * ks + 4 * half + vrow;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int col = dt * 32 + vcol;
        tr[ks][dt][0] = lds_read_tr16(Ob + bwd_tile_off<D>(r0, col));
        tr[ks][dt][1] = lds_read_tr16(Ob + bwd_tile_off<D>(r0 + 8, col));
        tr[ks][dt][2] = lds_read_tr16(Qb + bwd_tile_off<D>(r0, col));
        tr[ks][dt][3] = lds_read_tr16(Qb + bwd_tile_off<D>(r0 + 8, col));
      }
    }
    // dx = P (dP - Delta)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      pn = mfma32(oa[s], vb[s], pn);
#pragma unroll
      for (int r = s * PC; r < (s + 1) * PC; ++r) pa[r] = sa[r] * (pa[r] - d4[r / 4][r % 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pb[2], xb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[ks][e] = f2bf(sa[8 * ks + e]);
        xb[ks][e] = f2bf(pa[8 * ks + e]);
      }
    // dV^T += dO^T P over this wave's 32 rows (2 k-steps of 16)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 ao = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tr[ks][dt][0], tr[ks][dt][1], 0, 1, 2, 3, 4, 5, 6, 7));
        dva[dt] = mfma32(ao, pb[ks], dva[dt]);
      }
    // dK^T += Q^T dx
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 aq = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tr[ks][dt][2], tr[ks][dt][3], 0, 1, 2, 3, 4, 5, 6, 7));
        dka[dt] = mfma32(aq, xb[ks], dka[dt]);
      }
    if constexpr (MODE == 2) {
      // dL_j += sum over this wave's rows of dr_t q_t, from the transposed Q fragments (rows in
      // the same permuted order as the P registers); both key tiles' waves hold them, so each
      // takes half of the d tiles
      const float* Rb = Lb + 2 * kBlock;
      auto dl_tiles = [&](int dt0) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f32x4 r0 = *reinterpret_cast<const f32x4*>(&Rb[tb + 16 * ks]);
          const f32x4 r1 = *reinterpret_cast<const f32x4*>(&Rb[tb + 16 * ks + 8]);
#pragma unroll
          for (int dt = dt0; dt < dt0 + DT / 2; ++dt) {
            const bf16x4 q0 = __builtin_bit_cast(bf16x4, tr[ks][dt][2]);
            const bf16x4 q1 = __builtin_bit_cast(bf16x4, tr[ks][dt][3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dla[dt] = fmaf(bf2f(q0[e]), r0[e], dla[dt]);
              dla[dt] = fmaf(bf2f(q1[e]), r1[e], dla[dt]);
            }
          }
        }
      };
      if (kh == 0) dl_tiles(0);
      else dl_tiles(DT / 2);
    }
    sa = sn;
    pa = pn;
  }
  __syncthreads();   // stages free (the last wait was vmcnt(0))

  // sum the two row halves: waves th = 1 hand their accumulators to waves th = 0
  float* red = reinterpret_cast<float*>(smem);
  constexpr int RED = 2 * DT * 16 * kWave;       // floats per key half
  float dlv[DT];
  if constexpr (MODE == 2) {
    // dL: lanes l and l^32 hold the same columns for different rows
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dlv[dt] = wave_sum_xor32(dla[dt]);
  }
  if (th == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        red[kh * RED + (dt * 16 + i) * kWave + lane] = dka[dt][i];
        red[kh * RED + ((DT + dt) * 16 + i) * kWave + lane] = dva[dt][i];
      }
    if constexpr (MODE == 2) {
      if (half == 0)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          if (dt / (DT / 2) == kh) Lred[dt * 32 + l32] = dlv[dt];
    }
  }
  __syncthreads();
  if constexpr (MODE == 2) {
    // the two row halves of dL_j: written directly for a single work item, else as a partial
    if (th == 0 && half == 0)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        if (dt / (DT / 2) == kh) {
          const int d = dt * 32 + l32;
          const float val = dlv[dt] + Lred[d];
          if (nch == 1) dlm[((size_t)bg * NB + j) * D + d] = val * scale;
          else partL[((size_t)bg * max_work + wi) * D + d] = val;
        }
  }
  constexpr int FP = D + 4;                      // row pitch (floats) of the [key][d] tiles
  float* F = red + 2 * RED;                      // [2][64][FP]: dK then dV
  if (th == 0) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = dt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        const int u = kh * 32 + l32;
        F[u * FP + d] = dka[dt][i] + red[kh * RED + (dt * 16 + i) * kWave + lane];
        F[kBlock * FP + u * FP + d] = dva[dt][i] + red[kh * RED + ((DT + dt) * 16 + i) * kWave + lane];
      }
  }
  __syncthreads();
  // write: bf16 dk, dv when this is the key block's only work item, else a float32 partial
  constexpr int ITEMS = 2 * kBlock * C;          // (which, key, 8 columns)
  for (int it = tid; it < ITEMS; it += 256) {
    const int which = it / (kBlock * C);
    const int u = (it / C) % kBlock, c8 = it % C;
    const float* src = F + which * kBlock * FP + u * FP + c8 * 8;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(src + 4);
    if (nch == 1) {
      const int tok = j * kBlock + u;
      if (tok < T) {
        const float sc = which == 0 ? scale : 1.0f;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = f2bf(a0[e] * sc);
          o[4 + e] = f2bf(a1[e] * sc);
        }
        bf16* dst = which == 0 ? dk : dv;
        *reinterpret_cast<bf16x8*>(dst + kvbase + (size_t)tok * D + c8 * 8) = o;
      }
    } else {
      float* pt = part + (((size_t)bg * max_work + wi) * 2 + which) * kBlock * D + u * D + c8 * 8;
      *reinterpret_cast<f32x4*>(pt) = a0;
      *reinterpret_cast<f32x4*>(pt + 4) = a1;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dk, dv of a key block with several work items (or none): partials summed in order
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ part,
                                                         const int* __restrict__ chunk_off,
                                                         bf16* __restrict__ dk,
                                                         bf16* __restrict__ dv,
                                                         const float* __restrict__ partL,
                                                         float* __restrict__ dlm, int Hkv, int T,
                                                         int NB, int max_work, float scale) {
  constexpr int C = D / 8;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * Hkv + g;
  const int c0 = chunk_off[(size_t)bg * (NB + 1) + j];
  const int c1 = chunk_off[(size_t)bg * (NB + 1) + j + 1];
  if (c1 - c0 == 1) return;                      // written by its only work item
  if (dlm != nullptr && threadIdx.x < D) {
    float acc = 0.0f;
    for (int chn = c0; chn < c1; ++chn) acc += partL[((size_t)bg * max_work + chn) * D + threadIdx.x];
    dlm[((size_t)bg * NB + j) * D + threadIdx.x] = acc * scale;
  }
  for (int it = threadIdx.x; it < 2 * kBlock * C; it += 256) {
    const int which = it / (kBlock * C);
    const int u = (it / C) % kBlock, c8 = it % C;
    const int tok = j * kBlock + u;
    if (tok >= T) continue;
    f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
    for (int chn = c0; chn < c1; ++chn) {
      const float* pt = part + (((size_t)bg * max_work + chn) * 2 + which) * kBlock * D + u * D + c8 * 8;
      a0 += *reinterpret_cast<const f32x4*>(pt);
      a1 += *reinterpret_cast<const f32x4*>(pt + 4);
    }
    const float sc = which == 0 ? scale : 1.0f;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = f2bf(a0[e] * sc);
      o[4 + e] = f2bf(a1[e] * sc);
    }
    bf16* dst = which == 0 ? dk : dv;
    *reinterpret_cast<bf16x8*>(dst + ((size_t)bg * T + tok) * D + c8 * 8) = o;
  }
}

// ---------------------------------------------------------------------------------------------
// selector-score gradient of each attended-set row (SAS)
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dsc_kernel(const int32_t* __restrict__ idx,
                                                      const float* __restrict__ sc,
                                                      const float* __restrict__ dg,
                                                      float* __restrict__ dsc, int R, int NA,
                                                      int64_t nrows, int mode) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= nrows) return;
  const int c = (int)(row % R);
  const int32_t* ir = idx + row * NA;
  const float* sr = sc ? sc + row * NA : nullptr;
  float* out = dsc + row * NA;
  int nval = 0;
  while (nval < NA && ir[nval] >= 0) ++nval;
  int ic = -1;
  for (int a = 0; a < nval; ++a)
    if (ir[a] == c) ic = a;
  float acc_c = 0.0f;
  for (int a = 0; a < NA; ++a) {
    float d = 0.0f;
    if (mode == 1 && a < nval && a != ic && ic >= 0) {
      const float sg = 1.0f / (1.0f + expf(sr[a] - sr[ic]));   // sigmoid(S_c - S_j)
      d = dg[row * NA + a] * sg;
      acc_c -= d;
    }
    out[a] = d;
  }
  if (ic >= 0 && mode == 1) out[ic] = acc_c;
}

// ---------------------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------------------
template <int D>
static hipError_t launch_backward_d(const Shape& s, const void* q, const void* k, const void* v,
                                    const void* lm, const int32_t* idx, const float* sc,
                                    const void* out, const float* lse, const void* dout, void* dq,
                                    void* dk, void* dv, float* dsc, float* dlm, void* ws,
                                    hipStream_t st) {
  BwdWs W;
  bwd_layout(s, (char*)ws, &W);
  const int BG = s.B * s.Hkv;
  const int64_t rows = (int64_t)s.B * s.Hq * s.Tq;
  const int64_t n_entries = (int64_t)BG * s.R * s.NA;
  const int mw = bwd_max_work(s);
  const float sl2 = s.scale * kLog2e;
  if (s.mode != 2) {
    constexpr int RPB = 4 * (kWave / (D / 8));
    hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       st, (const bf16*)out, (const bf16*)dout, W.delta, rows);
  }
  hipLaunchKernelGGL(bwd_fill_zero_kernel, dim3(1024), dim3(256), 0, st, W.cnt_off,
                     (int64_t)BG * (s.NB + 1), W.dg, n_entries);
  const unsigned eg = (unsigned)((n_entries + 255) / 256);
  hipLaunchKernelGGL(bwd_count_kernel, dim3(eg), dim3(256), 0, st, idx, W.cnt_off, s.R, s.NA,
                     s.NB, n_entries);
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(BG), dim3(1024), 0, st, W.cnt_off, W.cursor,
                     W.chunk_off, W.work, W.n_work, s.NB, mw);
  hipLaunchKernelGGL(bwd_fill_kernel, dim3(eg), dim3(256), 0, st, idx, W.cursor, W.list, s.R,
                     s.NA, s.NB, n_entries);
  hipLaunchKernelGGL(bwd_sort_kernel, dim3(s.NB, BG), dim3(256), 0, st, W.cnt_off, W.list, s.R,
                     s.NA, s.NB);
  const int hpw = (s.G % 4 == 0) ? 4 : (s.G % 2 == 0) ? 2 : 1;
  const int n_hc = s.G / hpw;
#define BSA_DQ(MODE, HPW)                                                                        \
  hipLaunchKernelGGL((bwd_dq_kernel<D, MODE, HPW>), dim3(s.R, s.Hkv * n_hc, s.B), dim3(HPW * 128),\
                     0, st, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,     \
                     lse, W.delta, idx, sc, (const bf16*)lm, (bf16*)dq, W.dg, W.gates, W.hstat,    \
                     W.hs_n, s.Hq, s.Hkv, s.G, s.Tq, s.R, s.NA, n_hc, sl2, s.scale)
#define BSA_DQ_H(MODE)                                           \
  if (hpw == 4) BSA_DQ(MODE, 4);                                  \
  else if (hpw == 2) BSA_DQ(MODE, 2);                             \
  else BSA_DQ(MODE, 1);
  if (s.mode == 1) {
    BSA_DQ_H(1)
  } else if (s.mode == 2) {
    BSA_DQ_H(2)
  } else {
    BSA_DQ_H(0)
  }
#undef BSA_DQ_H
#undef BSA_DQ
#define BSA_KV(MODE)                                                                            \
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, MODE>), dim3(mw, s.Hkv, s.B), dim3(256), 0, st,        \
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse,     \
                     W.delta, W.gates, W.cnt_off, W.chunk_off, W.list, W.work, W.n_work, W.part, \
                     (bf16*)dk, (bf16*)dv, W.hstat, W.hs_n, W.partL, dlm, s.Hq, s.Hkv, s.G,      \
                     s.Tq, s.R, s.NB, s.NA, mw, sl2, s.scale)
  if (s.mode == 1) BSA_KV(1);
  else if (s.mode == 2) BSA_KV(2);
  else BSA_KV(0);
#undef BSA_KV
  hipLaunchKernelGGL(bwd_reduce_kernel<D>, dim3(s.NB, s.Hkv, s.B), dim3(256), 0, st, W.part,
                     W.chunk_off, (bf16*)dk, (bf16*)dv, W.partL, s.mode == 2 ? dlm : nullptr,
                     s.Hkv, s.Tq, s.NB, mw, s.scale);
  if (dsc != nullptr)
    hipLaunchKernelGGL(bwd_dsc_kernel, dim3((unsigned)((BG * (int64_t)s.R + 255) / 256)), dim3(256),
                       0, st, idx, sc, W.dg, dsc, s.R, s.NA, (int64_t)BG * s.R, s.mode);
  return hipGetLastError();
}

hipError_t launch_attend_backward(const Shape& s, const void* q, const void* k, const void* v,
                                  const void* lm, const int32_t* idx, const float* sc,
                                  const void* out, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, float* dsc, float* dlm, void* ws,
                                  hipStream_t st) {
  if (s.D == 128)
    return launch_backward_d<128>(s, q, k, v, lm, idx, sc, out, lse, dout, dq, dk, dv, dsc, dlm, ws, st);
  return launch_backward_d<64>(s, q, k, v, lm, idx, sc, out, lse, dout, dq, dk, dv, dsc, dlm, ws, st);
}

}  // namespace bsa
