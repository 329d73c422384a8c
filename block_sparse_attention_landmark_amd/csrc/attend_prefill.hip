// Block-sparse attention over the attended block lists: bf16 prefill kernels.
//
// PLAIN / SAS: softmax over the keys of the attended blocks (causal inside the current
// block), computed FlashAttention-style, block by block with a running max and sum and no
// materialised score matrix (SAS page, summary paragraph 4: the kernel works block-wise without
// building the full square matrix).  SAS adds g_j = log sigmoid(S_j - S_c) to every logit of
// block j != c, inside the softmax (SAS page, summary paragraph 3, "Key facts" item 3).
//
// HiLS: every query attends to each attended chunk separately; the per-chunk results are merged
// with weights softmax_j(q . L_j / sqrt(D)) over the attended chunks (HiLS page, summary
// paragraph 2: per-chunk attention combined by the chunks' retrieval scores).
//
// bf16 prefill: one workgroup per (batch, kv group, query block, head chunk) holds up to four
// query heads x 64 tokens (two waves per head, 32 query rows per wave), so every gathered K/V
// block in LDS feeds up to 256 query rows.  Scores are computed transposed, S^T = K Q^T, on
// 32x32x16 bf16 MFMA so that each lane owns one query row: the row max and sum need only the
// lane's own registers and one exchange with the lane 32 apart.  P V is computed as
// O^T = V^T P^T with P taken straight from the score registers (the contraction order over
// keys is permuted identically on both operands), V transposed into LDS when staged.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "attend_common.hpp"
#include "bsa_internal.hpp"

namespace bsa {

// =============================================================================================
// bf16 prefill
// =============================================================================================
// Pipeline per workgroup: the K and V blocks of attended entry a+1 are written from registers
// into the second LDS buffer and the global loads of entry a+2 are issued while the waves finish
// entry a, so each block costs one barrier and its HBM/L2 latency hides behind a block of math.
// V stays row-major in LDS and reaches the P V MFMA through transposed LDS reads.
//
// Softmax (PLAIN/SAS), per query row, in log2 units: the block's max comes from the raw scores
// (the scale is positive and the gate constant per block), every probability is one FMA and
// one exp2, and the running max is only raised -- rescaling O and the sum -- when the block's
// max exceeds it by more than 8 (probabilities then stay below 2^8, far inside float32 and bf16
// range); the final O / sum is unchanged by the choice of reference max.
constexpr float kLazyRescale = 8.0f;
constexpr float kPpSumLimit = 65536.0f;   // see the vector phase of the ping-pong kernel
constexpr int kPpUnits = 4;       // staging units in LDS for the ping-pong prefill kernel (a power
                                   // of two keeps the unit addressing cheap)

// WIDE (HiLS with more than 64 attended entries): the merge weights are taken 64 entries at a
// time, the table refreshed inside the entry loop; the common case keeps that code out of it.
template <int D, int MODE, int HPW, bool WIDE>
__global__ __launch_bounds__(HPW * 128) void attend_prefill_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ lm, const int32_t* __restrict__ idx, const float* __restrict__ sc,
    bf16* __restrict__ out, float* __restrict__ lse, int Hq, int Hkv, int G, int T, int NQB,
    int NA, int n_hc, float scale_log2) {
  constexpr int NWAVE = HPW * 2;
  constexpr int NT = NWAVE * kWave;
  constexpr int KP = D + 8;        // K tile row pitch (elements)
  constexpr int VP = D + 32;       // V tile row pitch (elements): rows 16 banks apart, so the
                                   // transposed reads of 32 lanes cover all 64 banks once
  constexpr int C8 = D / 8;        // 16-byte chunks per row
  constexpr int CPT = kBlock * C8 / NT;   // chunks of each tile staged per thread
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][kBlock * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][kBlock * VP];
  __shared__ float wbuf[MODE == 2 ? NWAVE * 64 * 32 : 1];

  // Order: kv group major, query blocks (heavy, late ones first) minor.  Workgroups are dealt
  // round-robin over the 8 XCDs, so all XCDs work on the same kv group at a time and share its
  // K/V blocks through the memory-side cache instead of each streaming a different group.
  const int nh = Hkv * n_hc;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int b = lin / (NQB * nh);
  const int rem = lin % (NQB * nh);
  const int gh = rem / NQB;
  const int c = NQB - 1 - rem % NQB;          // heavy (late) query blocks first
  const int g = gh / n_hc;
  const int hc = gh % n_hc;

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const int h = g * G + hc * HPW + w / 2;
  const int tq = c * kBlock + (w % 2) * 32 + l32;
  const bool row_ok = tq < T;

  bf16x8 qf[D / 16];
  {
    const bf16* qrow = q + ((size_t)(b * Hq + h) * T + min(tq, T - 1)) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * half);
      if (!row_ok) raw = u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const size_t kvbase = (size_t)(b * Hkv + g) * T * D;
  const size_t rowsel = ((size_t)(b * Hkv + g) * NQB + c) * NA;
  const int32_t* irow = idx + rowsel;
  const float* srow = sc + rowsel;
  const int nval = count_valid(irow, NA);
  float s_ref = 0.0f;
  if (MODE == 1 && nval > 0) s_ref = srow[nval - 1];

  // ---- staging helpers ----
  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int a) {
    const int j = irow[a];
    const bool ok = j >= 0 && j <= c;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + i * NT;
      const int row = ci / C8, c8 = ci % C8;
      const int tok = j * kBlock + row;
      kreg[i] = u32x4{0u, 0u, 0u, 0u};
      vreg[i] = u32x4{0u, 0u, 0u, 0u};
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
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KP + c8 * 8]) = kreg[i];
      *reinterpret_cast<u32x4*>(&Vs[buf][row * VP + c8 * 8]) = vreg[i];
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // HiLS: retrieval logits (log2 units) of the entries e0 .. e0+63 for this wave's 32 query rows
  // (-inf past nval): R^T = L Q^T on MFMA; register i of tile kt holds entry
  // e0 + kt*32 + 8*(i/4) + 4*half + i%4.  The landmark rows of the first 64 entries are staged in
  // LDS once (from_lds); those of later entries are read straight from memory as A fragments.
  float w_max = 0.0f, w_inv = 0.0f;            // HiLS: the rows' max logit and 1 / sum
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
          a = *reinterpret_cast<const bf16x8*>(&Ks[1][(kt * 32 + l32) * KP + 16 * s + 8 * half]);
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
  // the weights w_j = 2^(r_j - max) / sum of the entries in rt into this wave's table
  auto hils_weights = [&](const f32x16* rt) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        wbuf[(w * 64 + slot) * 32 + l32] = fast_exp2(rt[kt][i] - w_max) * w_inv;
      }
  };

  if (nval > 0) load_tile(0);

  if constexpr (MODE == 2) {
    // landmark rows of the first 64 entries, staged in the second K buffer (which the pipeline
    // first writes after the next barrier)
    for (int ci = tid; ci < kBlock * C8; ci += NT) {
      const int row = ci / C8, c8 = ci % C8;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      const int jr = row < nval ? irow[row] : -1;
      if (jr >= 0 && jr <= c)
        val = *reinterpret_cast<const u32x4*>(lm + ((size_t)(b * Hkv + g) * NQB + jr) * D + c8 * 8);
      *reinterpret_cast<u32x4*>(&Ks[1][row * KP + c8 * 8]) = val;
    }
    __syncthreads();
    // softmax of the retrieval logits over every attended chunk, 64 entries at a time: the max
    // and the sum are carried from one group of 64 to the next (one group: a plain max and sum)
    const int ngr = WIDE ? (nval + 63) / 64 : min(nval, 1);
    f32x16 rt[2];
    float den = 0.0f;
    w_max = -INFINITY;
    for (int gi = 0; gi < ngr; ++gi) {
      hils_logits(gi * 64, rt, !WIDE || gi == 0);
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
      if (WIDE && ngr > 1) hils_logits(0, rt, true);
      hils_weights(rt);
    }
  }

  if (nval > 0) store_tile(0);
  if (nval > 1) load_tile(1);
  __syncthreads();
  float gvec = 0.0f;        // SAS gates (log2 units) of entries gbase .. gbase + 63, one per lane
  int gbase = -kWave;

  for (int a = 0; a < nval; ++a) {
    const int buf = a & 1;
    const int j = irow[a];
    if constexpr (MODE == 2 && WIDE) {
      if (a > 0 && a % 64 == 0) {               // the weights of the next 64 entries
        f32x16 rt[2];
        hils_logits(a, rt, false);
        hils_weights(rt);
      }
    }
    if (j >= 0 && j <= c) {
      const bf16* Kb = Ks[buf];
      const bf16* Vb = Vs[buf];
      // S^T = K Q^T: st[kt][i] = score of key kt*32 + 8*(i/4) + 4*half + i%4 for query row l32
      // all K fragments first, so the MFMAs do not each wait on their own LDS read
      bf16x8 kf[2][D / 16];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          kf[kt][s] = *reinterpret_cast<const bf16x8*>(&Kb[(kt * 32 + l32) * KP + 16 * s + 8 * half]);
      f32x16 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) st[kt][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) st[kt] = mfma32(kf[kt][s], qf[s], st[kt]);
      }
      // schedule: every K-fragment read, then the MFMAs (the reads of the second key tile land
      // while the first tile's MFMAs run)
      __builtin_amdgcn_sched_group_barrier(0x100, D / 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, D / 8, 0);
      float mx = -INFINITY;
      if (j == c) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
            if (j * kBlock + key > tq) st[kt][i] = -INFINITY;
            mx = fmaxf(mx, st[kt][i]);
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kt][i]);
      }
      mx = wave_max_xor32(mx);
      if constexpr (MODE == 2) {
        const float mj = mx * scale_log2;
        float lsum = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = fast_exp2(fmaf(st[kt][i], scale_log2, -mj));
            st[kt][i] = e;
            lsum += e;
          }
        const float lj = wave_sum_xor32(lsum);
        const float coef = wbuf[(w * 64 + a % 64) * 32 + l32] / lj;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) st[kt][i] *= coef;
      } else {
        float gate2 = 0.0f;
        if constexpr (MODE == 1) {
          // gates of 64 entries at a time, one per lane; this entry's is read from its lane
          if (a >= gbase + kWave) {
            gbase = a;
            const int e = gbase + lane;
            gvec = 0.0f;
            if (e < nval && irow[e] != c) gvec = log_sigmoid(srow[e] - s_ref) * kLog2e;
          }
          gate2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gvec), a - gbase));
        }
        const float m_blk = fmaf(mx, scale_log2, gate2);
        const bool need = m_blk > m_run + kLazyRescale;
        if (__any(need)) {
          const float m_new = need ? m_blk : m_run;
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        }
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
        l_run += lsum;
      }
      // O^T += V^T P^T over 4 k-steps of 16 keys; lane half h supplies keys
      // 16ks + 4h + {0..3} and 16ks + 8 + 4h + {0..3} (same order in both operands)
      const int vrow = (lane % 16) / 4;
      const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = f2bf(st[ks / 2][8 * (ks % 2) + e]);
        const bf16* v0 = Vb + (16 * ks + 4 * half + vrow) * VP + vcol;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const i16x4 x0 = lds_read_tr16(v0 + dt * 32);
          const i16x4 x1 = lds_read_tr16(v0 + 8 * VP + dt * 32);
          const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[dt] = mfma32(av, pb, o[dt]);
        }
      }
    }
    if (a + 1 < nval) store_tile(buf ^ 1);
    if (a + 2 < nval) load_tile(a + 2);
    __syncthreads();
  }

  float inv = 1.0f;
  float lse_val = 0.0f;
  if constexpr (MODE != 2) {
    const float l_tot = wave_sum_xor32(l_run);
    inv = 1.0f / l_tot;
    lse_val = (m_run + log2f(l_tot)) * kLn2;
  }
  if (row_ok) {
    bf16* orow = out + ((size_t)(b * Hq + h) * T + tq) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = f2bf(o[dt][4 * i4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * i4 + 4 * half) = ov;
      }
    if (MODE != 2 && lse != nullptr && half == 0) lse[(size_t)(b * Hq + h) * T + tq] = lse_val;
  }
}
// ---------------------------------------------------------------------------------------------
// bf16 prefill, PLAIN / SAS, four query heads per workgroup: ping-pong schedule
// ---------------------------------------------------------------------------------------------
// The eight waves form two groups of four (waves 0-3 and 4-7; each SIMD holds one wave of each).
// A wave's work per attended entry a alternates a matrix phase M(a) -- O^T += V(a-1)^T P(a-1)^T
// and S^T(a) = K(a) Q^T, all MFMA and LDS reads -- and a vector phase V(a) -- the online softmax
// of S(a) into P(a), all VALU.  The second group runs one phase behind the first, so in every
// phase one wave of each SIMD multiplies while the other exponentiates, and the SIMD overlaps the
// two instead of alternating between them.  A barrier separates phases.
//
// LDS holds kPpUnits (4) staging units of 32 KB; unit a = {K of entry a, V of entry a-1} is read
// in phases 2a and 2a+1.  It is copied straight from memory into LDS (global_load_lds, 1 KB per
// instruction, no register round trip) AHEAD = kPpUnits - 1 = 3 units in advance: during phases
// 2a-6 and 2a-5, into the buffer of unit a-4, which was read for the last time in phase 2a-7.
// So units a+1, a+2 and a+3 may be in flight while unit a is read.  Every wave issues exactly
// SPW copy instructions per unit (half in each of the two phases), and the waits before a
// barrier count those instructions (vmcnt = SPW or 2*SPW left in flight): both numbers, the
// unit count and the even split, are what wait_units relies on.  16-byte chunks are
// XOR-swizzled per row so the K fragment reads and the transposed V reads are free of bank
// conflicts.
template <int D, int MODE>
__global__ __launch_bounds__(512) void attend_prefill_pp_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ sc, bf16* __restrict__ out,
    float* __restrict__ lse, int Hq, int Hkv, int G, int T, int NQB, int NA, int n_hc,
    float scale_log2) {
  constexpr int C16 = D / 8;                  // 16-byte chunks per row
  constexpr int RPI = kWave / C16;            // rows per 1 KB copy instruction
  constexpr int TILE = kBlock * D;            // elements of one K or V tile
  constexpr int HSL = kBlock / RPI;           // copy instructions per tile
  constexpr int SPW = 2 * HSL / 8;            // copy instructions per wave per unit
  static_assert(SPW % 2 == 0, "each wave copies as many K as V slabs");
  __shared__ __attribute__((aligned(16))) bf16 U[kPpUnits][2 * TILE];

  // Order: (batch, kv group) pairs one after another, so that all XCDs share one group's K/V
  // blocks through the memory-side cache; within a pair, workgroups are dealt round-robin over
  // the 8 XCDs and each XCD takes a contiguous run of query blocks, so the blocks that
  // neighbouring query blocks share (local window, sink, overlapping top-K choices) are reused
  // from that XCD's L2.
  const int nh = Hkv * n_hc;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  int pair, qb;
  if (NQB % 8 == 0) {
    const int per = NQB / 8, xcd = lin % 8, kk = lin / 8;
    pair = kk / per;
    qb = xcd * per + kk % per;
  } else {
    pair = lin / NQB;
    qb = lin % NQB;
  }
  const int b = pair / nh;
  const int gh = pair % nh;
  const int c = NQB - 1 - qb;                 // heavy (late) query blocks first
  const int g = gh / n_hc;
  const int hc = gh % n_hc;

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const bool lead = w < 4;                    // the leading group
  const int h = g * G + hc * 4 + w / 2;
  const int tq = c * kBlock + (w % 2) * 32 + l32;
  const bool row_ok = tq < T;
  auto swzk = [](int row) { return D == 128 ? row % 16 : (row / 2) % 8; };
  auto swzv = [](int row) { return D == 128 ? 4 * (row % 4) : 0; };

  bf16x8 qf[D / 16];
  {
    const bf16* qrow = q + ((size_t)(b * Hq + h) * T + min(tq, T - 1)) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * half);
      if (!row_ok) raw = u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const size_t kvbase = (size_t)(b * Hkv + g) * T * D;
  const size_t rowsel = ((size_t)(b * Hkv + g) * NQB + c) * NA;
  const int32_t* irow = idx + rowsel;
  const float* srow = sc + rowsel;
  const int nval = count_valid(irow, NA);

  // entries 0..63 one per lane (block index, SAS gate in log2 units); later ones re-read
  int jvec = lane < nval ? irow[lane] : -1;
  float gvec = 0.0f;
  float s_ref = 0.0f;
  if constexpr (MODE == 1) {
    if (nval > 0) s_ref = srow[nval - 1];
    if (lane < nval && jvec != c) gvec = log_sigmoid(srow[lane] - s_ref) * kLog2e;
  }
  auto entry = [&](int a) {          // block of entry a (a < nval), wave-uniform
    const int j = a < kWave ? __builtin_amdgcn_readlane(jvec, a) : irow[a];
    return (j >= 0 && j <= c) ? j : -1;
  };
  auto gate = [&](int a, int j) {
    if constexpr (MODE != 1) return 0.0f;
    if (j == c) return 0.0f;
    if (a < kWave) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gvec), a));
    return log_sigmoid(srow[a] - s_ref) * kLog2e;
  };

  // ---- staging: wave w copies K slabs w, w+8, .. and V slabs w, w+8, .. of a unit ----
  // Unit a = {K(entry a), V(entry a-1)}, 0 <= a <= nval; the halves that do not exist (V of
  // unit 0, K of unit nval) copy a neighbouring entry instead so that every unit costs each wave
  // exactly SPW copy instructions (the waits count them).
  // Source of lane `lane` of copy instruction i within a block: row crow[i] (a block row past the
  // end of the sequence reads the last row instead; its probability is zero), logical chunk
  // (physical ^ swizzle); the block's base address is wave-uniform.
  int crow[SPW / 2], kcol[SPW / 2], vcol_[SPW / 2];
#pragma unroll
  for (int i = 0; i < SPW / 2; ++i) {
    crow[i] = (w + 8 * i) * RPI + lane / C16;
    kcol[i] = ((lane % C16) ^ swzk(crow[i])) * 16;
    vcol_[i] = ((lane % C16) ^ swzv(crow[i])) * 16;
  }
  const char* kb = reinterpret_cast<const char*>(k + kvbase);
  const char* vb = reinterpret_cast<const char*>(v + kvbase);
  // This wave's part of unit a: SPW copies of 1 KB (K slab, V slab, K slab, ...), issued in two
  // halves: copies x with x % 2 == h for half h (K slabs, then V slabs).
  const uint32_t u_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)&U[0][0];
  // entries 0..63, one per lane: the block a copy reads (the entry's block, or the current
  // block for an invalid entry) and that block's last row inside the sequence.  The block's
  // byte offset is formed in 64 bits from the wave-uniform index (a 32-bit offset would wrap
  // past 2^32 bytes of one head's K or V).
  const int jcp = (jvec >= 0 && jvec <= c) ? jvec : c;
  const int cp_lim = T - 1 - jcp * kBlock;
  auto copy_half = [&](int a, int hv) {
    const uint32_t dst = u_lds + (uint32_t)(a % kPpUnits) * (2 * TILE * 2);
    const int ae = hv == 0 ? min(a, nval - 1) : max(a - 1, 0);
    int j, lim;
    if (ae < kWave) {
      j = __builtin_amdgcn_readlane(jcp, ae);
      lim = __builtin_amdgcn_readlane(cp_lim, ae);
    } else {
      j = entry(ae);
      j = j < 0 ? c : j;
      lim = T - 1 - j * kBlock;
    }
    const char* blk = (hv == 0 ? kb : vb) + (size_t)j * (size_t)(kBlock * D * 2);
    sync_copies_barrier();     // race-check build only (every wave issues every copy_half)
#pragma unroll
    for (int i = 0; i < SPW / 2; ++i) {
      const int sl = w + 8 * i;
      dma_lds<16>(blk, (uint32_t)(min(crow[i], lim) * (D * 2) + (hv == 0 ? kcol[i] : vcol_[i])),
                dst + (hv * TILE + sl * RPI * D) * 2);
    }
    sync_copies_barrier();
  };
  auto copy_unit = [&](int a) {
    copy_half(a, 0);
    copy_half(a, 1);
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
  f32x16 st[2];
  bf16x8 pf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[ks][e] = f2bf(0.0f);
  float m_run = -INFINITY, l_run = 0.0f;

  const int vrow = (lane % 16) / 4;
  const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);

  // matrix phase of entry a: O^T += V^T P^T for entry a-1 (PV) and S^T = K Q^T for entry a
  // (QK).  LDS reads run one MFMA group ahead of the MFMAs that consume them: the V fragments
  // of k-step ks+1 (or the first K fragments) load during the MFMAs of k-step ks, the second
  // key tile's K fragments during the first tile's MFMAs.
  auto mphase = [&](int a, auto pv_tag, auto qk_tag) {
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool QK = decltype(qk_tag)::value;
    const bf16* Ku = U[a % kPpUnits];
    const bf16* Vu = U[a % kPpUnits] + TILE;
    auto read_v = [&](int ks, bf16x8* vf) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int r0 = 16 * ks + 4 * half + vrow;
        const int col = dt * 32 + vcol;
        const bf16* p0 = Vu + r0 * D + (((col / 8) ^ swzv(r0)) * 8) + col % 8;
        const bf16* p1 = Vu + (r0 + 8) * D + (((col / 8) ^ swzv(r0 + 8)) * 8) + col % 8;
        const i16x4 x0 = lds_read_tr16(p0);
        const i16x4 x1 = lds_read_tr16(p1);
        vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto read_k = [&](int kt, bf16x8* kf) {
      const int row = kt * 32 + l32;
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        kf[s] = *reinterpret_cast<const bf16x8*>(Ku + row * D + (((2 * s + half) ^ swzk(row)) * 8));
    };
    bf16x8 kf[2][D / 16];
    if constexpr (PV) {
      bf16x8 vf[4][D / 32];
      read_v(0, vf[0]);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 32), 0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks < 3) read_v(ks + 1, vf[ks + 1]);
        else if (QK) read_k(0, kf[0]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] = mfma32(vf[ks][dt], pf[ks], o[dt]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (ks < 3 || QK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    } else {
      read_k(0, kf[0]);
      __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);
    }
    if constexpr (QK) {
      read_k(1, kf[1]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) st[kt][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) st[kt] = mfma32(kf[kt][s], qf[s], st[kt]);
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);
    }
  };

  // vector phase of entry a: online softmax of its scores into pf.  The probabilities are first
  // taken against the running reference max; only if some row's sum then exceeds kPpSumLimit
  // (the block holds scores far above the reference, or this is the row's first block, whose
  // reference is -inf) is the block max formed, O and the sum rescaled and the probabilities
  // recomputed.  Below the limit every probability is at most kPpSumLimit, far inside float32
  // and bf16 range, and the final O / sum does not depend on the reference.
  auto vphase = [&](int a) {
    const int j = entry(a);
    if (j < 0) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[kt][i] = -INFINITY;
    } else if (j == c) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
          if (j * kBlock + key > tq) st[kt][i] = -INFINITY;
        }
    }
    const float gate2 = gate(a, j);
    auto probs = [&](float bias) {
      float lsum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(st[ks / 2][8 * (ks % 2) + e], scale_log2, bias));
          lsum += p;
          pf[ks][e] = f2bf(p);
        }
      return lsum;
    };
    float lsum = probs(gate2 - m_run);
    if (__any(!(lsum <= kPpSumLimit))) {        // also true for inf / NaN sums
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kt][i]);
      mx = wave_max_xor32(mx);
      const float m_new = fmaxf(m_run, fmaf(mx, scale_log2, gate2));
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      lsum = probs(gate2 - m_run);
    }
    l_run += lsum;
  };

  // Phases (lead = waves 0-3, trail = waves 4-7; M = matrix phase, V = vector phase):
  //   0: lead M(0) QK only        1: lead V(0),   trail M(0) QK only
  //   2a: lead M(a), trail V(a-1)  2a+1: lead V(a), trail M(a)      (1 <= a < n)
  //   2n: lead M(n) PV only, trail V(n-1)      2n+1: trail M(n) PV only
  // Unit a+3 is copied during phases 2a and 2a+1 into the buffer of unit a-1 (read for the last
  // time in phase 2a-1): each wave issues half of its share after the MFMAs of its matrix phase
  // and half at the start of its vector phase, which spreads the copies over both phases.  Unit
  // a+1 is waited for at the end of phase 2a+1, so a copy has four to five phases to land.
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  constexpr int AHEAD = kPpUnits - 1;
  static_assert(AHEAD == 3, "the waits below count up to two units in flight");
  const int n = nval;
  // wait until at most `left` (0..2) units of copies are still in flight
  auto wait_units = [&](int left) {
    if (left >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * SPW));
    else if (left == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | SPW);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  if (n > 0) {
    // only unit 0 before the first phase: the copies of units 1..AHEAD-1 go out after the lead
    // group's first matrix phase (and while the trail group waits for it)
    copy_unit(0);
    wait_units(0);                              // unit 0 has landed
    __syncthreads();
    if (lead) mphase(0, F_{}, T_{});
    for (int u = 1; u < AHEAD && u <= n; ++u) copy_unit(u);
    if (AHEAD <= n) copy_half(AHEAD, 0);
    __syncthreads();
    if (lead) {
      if (AHEAD <= n) copy_half(AHEAD, 1);
      vphase(0);
    } else {
      mphase(0, F_{}, T_{});
      if (AHEAD <= n) copy_half(AHEAD, 1);
    }
    wait_units(min(AHEAD, n) - 1);              // unit 1 has landed
    __syncthreads();
    for (int a = 1; a < n; ++a) {
      const bool cp = a + AHEAD <= n;
      if (lead) {
        mphase(a, T_{}, T_{});
        if (cp) copy_half(a + AHEAD, 0);
      } else {
        if (cp) copy_half(a + AHEAD, 0);
        vphase(a - 1);
      }
      __syncthreads();
      if (lead) {
        if (cp) copy_half(a + AHEAD, 1);
        vphase(a);
      } else {
        mphase(a, T_{}, T_{});
        if (cp) copy_half(a + AHEAD, 1);
      }
      wait_units(min(a + AHEAD, n) - (a + 1));  // unit a+1 has landed
      __syncthreads();
    }
    if (lead) mphase(n, T_{}, F_{});
    else vphase(n - 1);
    __syncthreads();
    if (!lead) mphase(n, T_{}, F_{});
  }

  const float l_tot = wave_sum_xor32(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_val = (m_run + log2f(l_tot)) * kLn2;
  if (row_ok) {
    bf16* orow = out + ((size_t)(b * Hq + h) * T + tq) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = f2bf(o[dt][4 * i4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * i4 + 4 * half) = ov;
      }
    if (lse != nullptr && half == 0) lse[(size_t)(b * Hq + h) * T + tq] = lse_val;
  }
}

// =============================================================================================
// launchers
// =============================================================================================
template <int D>
static void launch_prefill_bf16_d(const Shape& s, const void* q, const void* k, const void* v,
                                  const void* lm, const int32_t* idx, const float* sc, void* out,
                                  float* lse, hipStream_t st) {
  const int hpw = (s.G % 4 == 0) ? 4 : (s.G % 2 == 0) ? 2 : 1;
  const int n_hc = s.G / hpw;
  dim3 grid(s.R, s.Hkv * n_hc, s.B);
  const float sl2 = s.scale * kLog2e;
#define BSA_PF(MODE, HPW, WIDE)                                                                \
  hipLaunchKernelGGL((attend_prefill_bf16_kernel<D, MODE, HPW, WIDE>), grid, dim3(HPW * 128), 0, \
                     st, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)lm, idx, sc, \
                     (bf16*)out, lse, s.Hq, s.Hkv, s.G, s.Tq, s.R, s.NA, n_hc, sl2)
#define BSA_PF_MODE(HPW)                          \
  if (s.mode == 0) BSA_PF(0, HPW, false);         \
  else if (s.mode == 1) BSA_PF(1, HPW, false);    \
  else if (s.NA > 64) BSA_PF(2, HPW, true);       \
  else BSA_PF(2, HPW, false);
#define BSA_PP(MODE)                                                                           \
  hipLaunchKernelGGL((attend_prefill_pp_kernel<D, MODE>), grid, dim3(512), 0, st,         \
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, idx, sc, (bf16*)out, lse, \
                     s.Hq, s.Hkv, s.G, s.Tq, s.R, s.NA, n_hc, sl2)
  if (hpw == 4 && s.mode == 0) {
    BSA_PP(0);
  } else if (hpw == 4 && s.mode == 1) {
    BSA_PP(1);
  } else if (hpw == 4) {
    BSA_PF_MODE(4)
  } else if (hpw == 2) {
    BSA_PF_MODE(2)
  } else {
    BSA_PF_MODE(1)
  }
#undef BSA_PF_MODE
#undef BSA_PF
#undef BSA_PP
}

hipError_t launch_attend_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                 const void* lm, const int32_t* idx, const float* sc, void* out,
                                 float* lse, hipStream_t st) {
  if (s.bf16) {
    if (s.D == 128) launch_prefill_bf16_d<128>(s, q, k, v, lm, idx, sc, out, lse, st);
    else launch_prefill_bf16_d<64>(s, q, k, v, lm, idx, sc, out, lse, st);
  } else {
    return launch_attend_f32(s, q, k, v, lm, idx, sc, out, lse, st);
  }
  return hipGetLastError();
}

}  // namespace bsa
