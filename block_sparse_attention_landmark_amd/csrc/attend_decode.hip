// Block-sparse attention over the attended block lists: bf16 decode kernels (one query token
// per sequence; the attended blocks of each (sequence, kv group) are streamed by one or more
// workgroups and the partial softmax states merged through their log-sum-exp).  Same PLAIN /
// SAS / HiLS rules as the prefill kernels.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "attend_common.hpp"
#include "bsa_internal.hpp"
#include "select_common.hpp"

namespace bsa {

// =============================================================================================
// bf16 decode: split-K over the attended blocks, one block per wave
// =============================================================================================
constexpr int kDecodeWaves = 4;          // waves per workgroup
constexpr int kMergeMaxSplits = 64;      // partial states merged per (sequence, kv group)

constexpr int kDecodeTargetWorkgroups = 256;   // one per CU is enough to stream the cache

// fused selection + attention: limits of the LDS-held score row and attended set
constexpr int kFusedMaxBlocks = 4096;
constexpr int kFusedMaxNA = 256;

// Splits of the attended blocks of one (sequence, kv group): as few as keep the GPU busy (each
// split's partial state costs a write and a read), at most kMergeMaxSplits.
inline int decode_nsplit(int NA, int pairs) {
  const int max_useful = (NA + kDecodeWaves - 1) / kDecodeWaves;
  const int want = (kDecodeTargetWorkgroups + pairs - 1) / pairs;
  return std::max(1, std::min(std::min(want, max_useful), kMergeMaxSplits));
}
inline int decode_blocks_per_wave(int NA, int nsplit) {
  const int per_split = (NA + nsplit - 1) / nsplit;
  return (per_split + kDecodeWaves - 1) / kDecodeWaves;
}

// One workgroup per (sequence, kv group, split); wave w of split s takes the attended entries
// (s * waves * bpw) + w + waves * i, i < bpw.  K and V blocks are copied straight from memory
// into the wave's LDS tiles (no register round trip, 1 KB per instruction), with 16-byte chunks
// XOR-swizzled so the fragment and transposed reads are free of bank conflicts.  Each wave keeps
// an online softmax state; the waves' states are combined in LDS and written as the split's
// partial state.
//
// PAGED: the cache is a pool of 64-token pages [n_pages, Hkv, 64, D]; block j of sequence b is
// page page_table[b * NB + j] (clamped into the pool) and the sequence holds seq_lens[b] tokens
// (clamped to 1 .. NB * 64); otherwise kc / vc are [B, Hkv, Tk, D] and every sequence holds Tk.
//
// FUSED (nsplit == 1): the workgroup first selects its own attended set -- the selector vector
// (sum of the group's query heads), the scores of blocks 0..c against the landmarks, the top-K
// with the forced sink and local blocks (the same arithmetic, bit for bit, as the decode
// selection kernel) -- writes it to sel_idx / sel_sc and attends it from LDS.  The sink and local
// blocks are processed first, and their copies are issued before the top-K runs, so the cache
// stream starts while the selection is still being decided.
template <int D, int MODE, bool PAGED, bool FUSED>
__global__ __launch_bounds__(kDecodeWaves * 64) void attend_decode_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const bf16* __restrict__ lm, const int32_t* __restrict__ idx, const float* __restrict__ sc,
    float* __restrict__ part_o, float* __restrict__ part_ml, bf16* __restrict__ out,
    float* __restrict__ lse, int Hq, int Hkv, int G, int Tk_all, int NB, int NA, int nsplit, int bpw,
    float scale_log2, const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    int n_pages, int32_t* __restrict__ sel_idx, float* __restrict__ sel_sc, int topk, int n_sink,
    int n_local) {
  constexpr int C16 = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / C16;              // rows covered by one 64-lane 16-byte copy
  __shared__ __attribute__((aligned(16))) bf16 Ks[kDecodeWaves][kBlock * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kDecodeWaves][kBlock * D];
  __shared__ float comb_ml[kDecodeWaves][32][2];
  __shared__ __attribute__((aligned(16))) bf16 Ls[kDecodeWaves][128];   // HiLS: landmark row

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const bool row_ok = l32 < G;
  const int h = g * G + min(l32, G - 1);
  const int Tk = PAGED ? min(max(seq_lens[b], 1), NB * kBlock) : Tk_all;   // this sequence
  const int c = (Tk - 1) / kBlock;
  // chunk swizzles (physical 16-byte chunk = logical ^ swz(row)): for the V tile, the four rows of
  // a transposed read land on distinct banks; for the K tile, the 16 rows of a fragment read do
  auto swz = [](int row) { return D == 128 ? 4 * (row % 4) : 0; };
  auto swzk = [](int row) { return D == 128 ? row % 16 : (row / 2) % 8; };

  bf16x8 qf[D / 16];
  {
    const bf16* qrow = q + (size_t)(b * Hq + h) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * half);
      if (!row_ok) raw = u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const size_t kvbase = (size_t)(b * Hkv + g) * Tk_all * D;
  // first element of block j of this (sequence, kv group) in kc / vc
  auto block_at = [&](int j) -> size_t {
    if constexpr (PAGED) {
      const int pg = min(max(page_table[(size_t)b * NB + j], 0), n_pages - 1);
      return ((size_t)pg * Hkv + g) * kBlock * D;
    } else {
      return kvbase + (size_t)j * kBlock * D;
    }
  };
  const int32_t* irow = FUSED ? nullptr : idx + (size_t)(b * Hkv + g) * NA;
  const float* srow = FUSED ? nullptr : sc + (size_t)(b * Hkv + g) * NA;
  int nval = FUSED ? 0 : count_valid(irow, NA);
  bf16* kt_ = Ks[w];
  bf16* vt = Vs[w];
  const uint32_t k_lds = lds_addr_of(kt_), v_lds = lds_addr_of(vt), l_lds = lds_addr_of(Ls[w]);
  const int vrow = (lane % 16) / 4;
  const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // copy the K (or V) rows of block j into this wave's tile, 1 KB per instruction (rows past
  // the cache end read its last row; their probabilities are zero); HiLS also copies the
  // block's landmark row beside the K tile
  auto copy_k = [&](int j) {
    const char* base = reinterpret_cast<const char*>(kc + block_at(j));
#pragma unroll
    for (int n = 0; n < kBlock / RPI; ++n) {
      const int row = n * RPI + lane / C16;
      const int r = min(row, Tk - 1 - j * kBlock);
      dma_lds<16>(base, (uint32_t)((r * D + ((lane % C16) ^ swzk(row)) * 8) * 2),
                  k_lds + (uint32_t)(n * RPI * D * 2));
    }
    if constexpr (MODE == 2) {
      const char* lrow = reinterpret_cast<const char*>(lm + ((size_t)(b * Hkv + g) * NB + j) * D);
      dma_lds<4>(lrow, (uint32_t)((lane % (D / 2)) * 4), l_lds);
    }
  };
  auto copy_v = [&](int j) {
    const char* base = reinterpret_cast<const char*>(vc + block_at(j));
#pragma unroll
    for (int n = 0; n < kBlock / RPI; ++n) {
      const int row = n * RPI + lane / C16;
      const int r = min(row, Tk - 1 - j * kBlock);
      dma_lds<16>(base, (uint32_t)((r * D + ((lane % C16) ^ swz(row)) * 8) * 2),
                  v_lds + (uint32_t)(n * RPI * D * 2));
    }
  };

  // ---- FUSED: select the attended set of this (sequence, kv group) into LDS ----
  int32_t* fidx = nullptr;      // the attended set in LDS (FUSED)
  float* fsc = nullptr;
  int n_forced = 0, n_sink_eff = 0;
  if constexpr (FUSED) {
    __shared__ float s_qb[D];
    __shared__ float s_score[kFusedMaxBlocks];
    __shared__ int s_hist[kTopkHistWords];
    __shared__ int s_sbuf[kDecodeWaves];
    __shared__ int s_sh[2];
    __shared__ int32_t s_idx[kFusedMaxNA];
    __shared__ float s_sel[kFusedMaxNA];
    fidx = s_idx;
    fsc = s_sel;
    const int tid = threadIdx.x;
    // selector vector: sum of the group's query heads (float64, then float32)
    if (tid < D) {
      double acc = 0.0;
      for (int hh = 0; hh < G; ++hh) acc += (double)bf2f(q[(size_t)(b * Hq + g * G + hh) * D + tid]);
      s_qb[tid] = (float)acc;
    }
    __syncthreads();
    // scores of blocks 0..c, one landmark row per lane: wave w streams rows
    // (4 r + w) * 64 .. +64 of round r straight into its own two tiles (rounds alternate between
    // them, two rounds in flight), 16-byte chunks XOR-swizzled by row so that the lanes' row
    // reads hit distinct banks; each lane then sums q . L over the row in dimension order
    {
      constexpr int C16 = D / 8;                // 16-byte chunks per row
      constexpr int RPI = kWave / C16;          // rows per copy instruction
      constexpr int NI = kBlock / RPI;          // copy instructions per 64-row round
      auto swzl = [](int row) { return D == 128 ? row % 16 : (row / 2) % 8; };
      const char* lrows = reinterpret_cast<const char*>(lm + (size_t)(b * Hkv + g) * NB * D);
      auto issue = [&](int r) {
        const int row0 = (r * kDecodeWaves + w) * kBlock;
        if (row0 > c) return;
        const uint32_t dst = (r & 1) ? v_lds : k_lds;
#pragma unroll
        for (int n = 0; n < NI; ++n) {
          const int row = n * RPI + lane / C16;
          const int rr = min(row0 + row, c);
          dma_lds<16>(lrows, (uint32_t)((rr * D + ((lane % C16) ^ swzl(row)) * 8) * 2),
                      dst + (uint32_t)(n * RPI * D * 2));
        }
      };
      issue(0);
      issue(1);
      for (int r = 0;; ++r) {
        const int row0 = (r * kDecodeWaves + w) * kBlock;
        if (row0 > c) break;
        if (row0 + kDecodeWaves * kBlock <= c)   // round r + 1 is in flight behind round r
          __builtin_amdgcn_s_waitcnt(0x0F70 | (NI & 15) | ((NI >> 4) << 14));
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);
        const bf16* tile = (r & 1) ? vt : kt_;
        const int row = row0 + lane;
        float sdot = 0.0f;
#pragma unroll
        for (int k = 0; k < C16; ++k) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(tile + lane * D + ((k ^ swzl(lane)) * 8));
#pragma unroll
          for (int e = 0; e < 8; ++e) sdot = fmaf(s_qb[8 * k + e], bf2f(x[e]), sdot);
        }
        if (row <= c) s_score[row] = sdot;
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this tile may be overwritten
        issue(r + 2);
      }
    }
    __syncthreads();
    // the forced blocks (sink, then the local window) are this set's first entries in the order
    // processed below; wave w < n_forced starts copying forced block w now
    n_sink_eff = min(n_sink, c + 1);
    const int loc_beg = max(n_sink, c - n_local + 1);
    n_forced = n_sink_eff + max(0, c - loc_beg + 1);
    if (w < n_forced) {
      const int jf = w < n_sink_eff ? w : loc_beg + (w - n_sink_eff);
      copy_k(jf);
      copy_v(jf);
    }
    topk_select<kDecodeWaves * 64>(
        [&](int jj) { return s_score[jj]; }, [&](int i) { return float_key(s_score[n_sink + i]); },
        c, topk, n_sink, n_local, NA, s_idx, s_sel, s_hist, s_sbuf, s_sh);
    __syncthreads();
    int32_t* gi = sel_idx + (size_t)(b * Hkv + g) * NA;
    float* gs = sel_sc + (size_t)(b * Hkv + g) * NA;
    for (int i = tid; i < NA; i += kDecodeWaves * 64) {
      gi[i] = s_idx[i];
      gs[i] = s_sel[i];
    }
    nval = n_forced + min(topk, max(0, c - n_local - n_sink + 1));
  }
  // position, in the attended-set row, of the entry processed p-th: the stored order unless
  // FUSED, where the forced blocks come first (sink entries, local entries, then the chosen)
  auto pos_of = [&](int p) {
    if constexpr (!FUSED) return p;
    const int kc_ = nval - n_forced;
    if (p < n_sink_eff) return p;
    if (p < n_forced) return kc_ + p;
    return p - (n_forced - n_sink_eff);
  };

  // This wave's entries: the p-th processed with p = a0 + waves * it for it < n_it.  They are
  // held one per lane, 64 at a time (block index and SAS gate), and read with readlane, so the
  // loop below issues no memory loads besides the tile copies: the only copy wait is the full
  // one at the top of an iteration.
  const int a0 = split * kDecodeWaves * bpw + w;
  const int n_it = a0 < nval ? min(bpw, (nval - a0 + kDecodeWaves - 1) / kDecodeWaves) : 0;
  float s_ref = 0.0f;
  if (MODE == 1 && nval > 0) s_ref = FUSED ? fsc[nval - 1] : srow[nval - 1];
  int ej = -1;
  float eg = 0.0f;
  auto load_batch = [&](int base) {
    const int it = base + lane;
    int jv = -1;
    float gv = 0.0f;
    if (it < n_it) {
      const int a = pos_of(a0 + kDecodeWaves * it);
      jv = FUSED ? fidx[a] : irow[a];
      if (jv < 0 || jv > c) jv = -1;
      else if (MODE == 1 && jv != c) gv = log_sigmoid((FUSED ? fsc[a] : srow[a]) - s_ref) * kLog2e;
    }
    ej = jv;
    eg = gv;
  };

  load_batch(0);
  int j = n_it > 0 ? __builtin_amdgcn_readlane(ej, 0) : -1;
  float gate2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(eg), 0));
  if (j >= 0 && !(FUSED && w < n_forced)) {    // (FUSED: forced blocks are already in flight)
    copy_k(j);
    copy_v(j);
  }
  for (int it = 0; it < n_it; ++it) {
    // the next entry (the held batch is reloaded at a 64-entry boundary: a full wait, rare)
    int jn = -1;
    float gn = 0.0f;
    if (it + 1 < n_it) {
      if (((it + 1) & 63) == 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        load_batch(it + 1);
      }
      jn = __builtin_amdgcn_readlane(ej, (it + 1) & 63);
      gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(eg), (it + 1) & 63));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): the tiles of block j have landed
    if (j < 0) {
      // an entry outside the causal range: nothing to attend; keep the copy stream going
      if (jn >= 0) {
        copy_k(jn);
        copy_v(jn);
      }
      j = jn;
      gate2 = gn;
      continue;
    }
    // S^T = K Q^T with K fragments (key kt*32 + l32, dims 16s + 8*half .. +8) read from LDS
    bf16x8 kf[2][D / 16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int row = kt * 32 + l32;
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        kf[kt][s] = *reinterpret_cast<const bf16x8*>(kt_ + row * D + (((2 * s + half) ^ swzk(row)) * 8));
    }
    float r2 = 0.0f;
    if constexpr (MODE == 2) {
      // retrieval score q . L_j of this lane's row, log2 units
      float part = 0.0f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 lv = *reinterpret_cast<const bf16x8*>(&Ls[w][16 * s + 8 * half]);
#pragma unroll
        for (int e = 0; e < 8; ++e) part += bf2f(qf[s][e]) * bf2f(lv[e]);
      }
      r2 = wave_sum_xor32(part) * scale_log2;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the K tile may be overwritten
    if (jn >= 0) copy_k(jn);
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) st[kt] = mfma32(kf[kt][s], qf[s], st[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        if (j * kBlock + key >= Tk) st[kt][i] = -INFINITY;
        mx = fmaxf(mx, st[kt][i]);
      }
    mx = wave_max_xor32(mx);
    float alpha, coef = 1.0f;
    if constexpr (MODE == 2) {
      // per-chunk softmax, then an online softmax over the chunks' retrieval scores
      float lsum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(fmaf(st[kt][i], scale_log2, -mx * scale_log2));
          st[kt][i] = e;
          lsum += e;
        }
      const float m_new = fmaxf(m_run, r2);
      alpha = fast_exp2(m_run - m_new);
      const float wr = fast_exp2(r2 - m_new);
      l_run = l_run * alpha + wr;
      m_run = m_new;
      coef = wr / wave_sum_xor32(lsum);
    } else {
      const float m_new = fmaxf(m_run, fmaf(mx, scale_log2, gate2));
      alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      const float bias = gate2 - m_run;
      float lsum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(st[kt][i], scale_log2, bias));
          st[kt][i] = p;
          lsum += p;
        }
      l_run = l_run * alpha + wave_sum_xor32(lsum);
    }
    if (alpha != 1.0f) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
    // O^T += V^T P^T; transposed reads of the swizzled V tile, all issued before the MFMAs
    bf16x8 vf[4][D / 32];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int r0 = 16 * ks + 4 * half + vrow;
        const int col = dt * 32 + vcol;               // element column (multiple of 4)
        const bf16* p0 = vt + r0 * D + (((col / 8) ^ swz(r0)) * 8) + col % 8;
        const bf16* p1 = vt + (r0 + 8) * D + (((col / 8) ^ swz(r0 + 8)) * 8) + col % 8;
        const i16x4 x0 = lds_read_tr16(p0);
        const i16x4 x1 = lds_read_tr16(p1);
        vf[ks][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the V tile may be overwritten
    if (jn >= 0) copy_v(jn);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = f2bf(st[ks / 2][8 * (ks % 2) + e] * coef);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] = mfma32(vf[ks][dt], pb, o[dt]);
    }
    j = jn;
    gate2 = gn;
  }

  // combine the waves' states (rows < G) through LDS (the K tiles are reused)
  __syncthreads();
  float* comb_o = reinterpret_cast<float*>(&Ks[0][0]);        // [wave][row][D]
  if (row_ok) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = o[dt][4 * i4 + e];
        *reinterpret_cast<f32x4*>(&comb_o[(w * 32 + l32) * D + dt * 32 + 8 * i4 + 4 * half]) = ov;
      }
    if (half == 0) {
      comb_ml[w][l32][0] = m_run;
      comb_ml[w][l32][1] = l_run;
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)(b * Hkv + g) * nsplit + split) * G;
  for (int e = threadIdx.x; e < G * D; e += kDecodeWaves * 64) {
    const int row = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kDecodeWaves; ++v) M = fmaxf(M, comb_ml[v][row][0]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int v = 0; v < kDecodeWaves; ++v) {
      const float m = comb_ml[v][row][0];
      if (m == -INFINITY) continue;
      const float f = fast_exp2(m - M);
      L += comb_ml[v][row][1] * f;
      acc += comb_o[(v * 32 + row) * D + d] * f;
    }
    if (nsplit == 1) {
      // a single split is the whole row: normalise and write the output directly
      const size_t orow = (size_t)b * Hq + g * G + row;
      out[orow * D + d] = f2bf(acc / L);
      if (MODE != 2 && lse != nullptr && d == 0) lse[orow] = (M + log2f(L)) * kLn2;
    } else {
      part_o[(pbase + row) * D + d] = acc;
      if (d == 0) {
        part_ml[(pbase + row) * 2 + 0] = M;
        part_ml[(pbase + row) * 2 + 1] = L;
      }
    }
  }
}

// Merge of the split partial states of one (sequence, kv group): every (row, split) pair loads
// its (m, l) at once, the per-split weights exp2(m_s - M) / L are formed in LDS, then each output
// element sums its column of partial outputs with independent loads.
template <typename OUT>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           OUT* __restrict__ out,
                                                           float* __restrict__ lse, int Hkv,
                                                           int G, int D, int nsplit,
                                                           int write_lse) {
  __shared__ float sm[32][kMergeMaxSplits];
  __shared__ float sl[32][kMergeMaxSplits];
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const size_t pb = (size_t)bg * nsplit;
  for (int t = threadIdx.x; t < G * nsplit; t += blockDim.x) {
    const int row = t / nsplit, s = t % nsplit;
    sm[row][s] = part_ml[((pb + s) * G + row) * 2];
    sl[row][s] = part_ml[((pb + s) * G + row) * 2 + 1];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int row = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, sm[row][s]);
    float L = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float f = (sm[row][s] == -INFINITY) ? 0.0f : fast_exp2(sm[row][s] - M);
      sm[row][s] = f;
      L += sl[row][s] * f;
    }
    const float inv = 1.0f / L;
    for (int s = 0; s < nsplit; ++s) sm[row][s] *= inv;
    if (write_lse && lse != nullptr) lse[(size_t)b * Hkv * G + g * G + row] = (M + log2f(L)) * kLn2;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int row = e / D, d = e % D;
    const float* col = part_o + (pb * G + row) * D + d;
    float acc = 0.0f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) acc += col[(size_t)s * G * D] * sm[row][s];
    out[((size_t)b * Hkv * G + g * G + row) * D + d] = (OUT)acc;
  }
}

// =============================================================================================
// static scratch for callers that cannot allocate
// =============================================================================================
// The split partial states of bsa_attend_decode_noalloc live in this file-scope array instead of
// a caller's workspace: each device that runs the library holds its own copy for the life of the
// process.  Host code never uses the array's name as an address: its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and kept below.  Every
// split writes its whole partial state before the merge reads it, so the array needs no
// clearing between calls; calls that overlap on one device share it and race.
constexpr int kScratchMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(hipStream_t st, void** ptr) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (st != nullptr) {
    e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// =============================================================================================
// launchers
// =============================================================================================
int decode_splits(const Shape& s) { return decode_nsplit(s.NA, s.B * s.Hkv); }

size_t decode_ws_bytes(const Shape& s) {
  if (!s.bf16 || decode_splits(s) == 1) return 0;
  const size_t rows = (size_t)s.B * s.Hkv * decode_splits(s) * s.G;
  const size_t o = (rows * s.D * sizeof(float) + 255) & ~(size_t)255;
  return o + rows * 2 * sizeof(float);
}

// FUSED: idx / sc are the outputs of the selection (sel_idx / sel_sc); nsplit is 1
template <int D, bool PAGED, bool FUSED>
static void launch_decode_bf16_d(const Shape& s, const void* q, const void* kc, const void* vc,
                                 const void* lm, const int32_t* idx, const float* sc, void* out,
                                 float* lse, void* ws, const Pages* pg, hipStream_t st) {
  const int nsplit = FUSED ? 1 : decode_splits(s);
  const size_t rows = (size_t)s.B * s.Hkv * nsplit * s.G;
  float* part_o = (float*)ws;
  float* part_ml =
      ws ? (float*)((char*)ws + ((rows * s.D * sizeof(float) + 255) & ~(size_t)255)) : nullptr;
  dim3 grid(nsplit, s.Hkv, s.B);
  const float sl2 = s.scale * kLog2e;
#define BSA_DEC(MODE)                                                                           \
  hipLaunchKernelGGL((attend_decode_bf16_kernel<D, MODE, PAGED, FUSED>), grid,                  \
                     dim3(kDecodeWaves * 64), 0, st, (const bf16*)q, (const bf16*)kc,           \
                     (const bf16*)vc, (const bf16*)lm, FUSED ? nullptr : idx,                   \
                     FUSED ? nullptr : sc, part_o, part_ml, (bf16*)out, lse, s.Hq, s.Hkv, s.G,  \
                     s.Tk, s.NB, s.NA, nsplit, decode_blocks_per_wave(s.NA, nsplit), sl2,       \
                     pg ? pg->table : nullptr, pg ? pg->lens : nullptr, pg ? pg->n_pages : 1,   \
                     FUSED ? const_cast<int32_t*>(idx) : nullptr,                              \
                     FUSED ? const_cast<float*>(sc) : nullptr, s.topk, s.n_sink, s.n_local)
  if (s.mode == 0) BSA_DEC(0);
  else if (s.mode == 1) BSA_DEC(1);
  else BSA_DEC(2);
#undef BSA_DEC
  if (!FUSED && nsplit > 1)
    hipLaunchKernelGGL(decode_merge_kernel<bf16>, dim3(s.B * s.Hkv), dim3(256), 0, st, part_o,
                       part_ml, (bf16*)out, lse, s.Hkv, s.G, s.D, nsplit, s.mode != 2 ? 1 : 0);
}

hipError_t launch_attend_decode(const Shape& s, const void* q, const void* kc, const void* vc,
                                const void* lm, const int32_t* idx, const float* sc, void* out,
                                float* lse, void* ws, hipStream_t st, const Pages* pg) {
  if (s.bf16) {
    if (pg != nullptr) {
      if (s.D == 128) launch_decode_bf16_d<128, true, false>(s, q, kc, vc, lm, idx, sc, out, lse, ws, pg, st);
      else launch_decode_bf16_d<64, true, false>(s, q, kc, vc, lm, idx, sc, out, lse, ws, pg, st);
    } else {
      if (s.D == 128) launch_decode_bf16_d<128, false, false>(s, q, kc, vc, lm, idx, sc, out, lse, ws, nullptr, st);
      else launch_decode_bf16_d<64, false, false>(s, q, kc, vc, lm, idx, sc, out, lse, ws, nullptr, st);
    }
  } else {
    return launch_attend_f32(s, q, kc, vc, lm, idx, sc, out, lse, st);
  }
  return hipGetLastError();
}

bool decode_step_fused(const Shape& s) {
  return s.bf16 && s.decode && decode_splits(s) == 1 && s.NB <= kFusedMaxBlocks &&
         s.NA <= kFusedMaxNA && s.G <= 32;
}

hipError_t launch_decode_step_fused(const Shape& s, const void* q, const void* kc, const void* vc,
                                    const void* lm, int32_t* idx, float* sc, void* out,
                                    float* lse, hipStream_t st, const Pages* pg) {
  if (pg != nullptr) {
    if (s.D == 128) launch_decode_bf16_d<128, true, true>(s, q, kc, vc, lm, idx, sc, out, lse, nullptr, pg, st);
    else launch_decode_bf16_d<64, true, true>(s, q, kc, vc, lm, idx, sc, out, lse, nullptr, pg, st);
  } else {
    if (s.D == 128) launch_decode_bf16_d<128, false, true>(s, q, kc, vc, lm, idx, sc, out, lse, nullptr, nullptr, st);
    else launch_decode_bf16_d<64, false, true>(s, q, kc, vc, lm, idx, sc, out, lse, nullptr, nullptr, st);
  }
  return hipGetLastError();
}

}  // namespace bsa
