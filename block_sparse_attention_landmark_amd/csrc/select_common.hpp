// Workgroup top-K of one selection row (shared by the selection kernels and the fused decode
// kernel).  Selection rule (SAS page, summary paragraph 1 and "How to apply": hard top-K; LSA
// page, first section, paragraph 4: the start of the context and a recent window are always
// added; SAS page, summary paragraph 3: the current block is always kept): among the candidate
// blocks n_sink <= j <= c - n_local, the K highest scores, lower block index first among equal
// scores, found by a 4-pass 8-bit radix select on order-preserving score keys and written in
// index order by a compaction.
#pragma once

#include "bsa_common.hpp"

namespace bsa {

// inclusive prefix sum over the 64 lanes of a wave: a Hillis-Steele scan inside each row of 16
// lanes with DPP row shifts, then the running totals carried across rows with DPP row
// broadcasts (lane 15 of a row to the next row, lane 31 to the upper half)
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x % kWave;
  const int r = lane % 16;
  int t = __builtin_amdgcn_mov_dpp(x, 0x111, 0xf, 0xf, false);   // row_shr:1
  if (r >= 1) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x112, 0xf, 0xf, false);       // row_shr:2
  if (r >= 2) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x114, 0xf, 0xf, false);       // row_shr:4
  if (r >= 4) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x118, 0xf, 0xf, false);       // row_shr:8
  if (r >= 8) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x142, 0xf, 0xf, false);       // row_bcast:15
  if (lane % 32 >= 16) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x143, 0xf, 0xf, false);       // row_bcast:31
  if (lane >= 32) x += t;
  return x;
}

// exclusive prefix sum over the workgroup; *total receives the sum of all x
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* sbuf, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  const int incl = wave_inclusive_scan(x);
  if (lane == kWave - 1) sbuf[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int v = sbuf[i];
    base += (i < w) ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

// Writes the attended set of query block c: forced sink entries, the K chosen candidates in
// ascending block order, the local window, -1 padding; osc gets the aligned scores.
// score_at(j) gives the score of block j <= c; key_at(i) the order-preserving key of candidate
// n_sink + i.  hist holds kTopkHistWords * R ints, sbuf NT / 64 and sh 2.  Rows of at most
// NT * KPT candidates keep every key in registers.  With R > 1 each digit is counted in R words
// (lane % R picks one; consecutive words, so distinct banks): the leading digits of a long row's
// keys are mostly equal, and a single word would serialise its thousands of increments.  Every
// thread of the workgroup must call it.
//
// The select is latency-bound (a few thousand keys per workgroup), so each radix pass costs two
// barriers: the digit counts go into one of two histograms while the other is cleared for the
// next pass, and the first wave alone finds the digit that holds the K-th key (four digits per
// lane, one wave scan).  The compaction takes one scan of (greater, equal) counts packed in one
// word when the row has fewer than 2^15 candidates.
constexpr int kTopkHistWords = 2 * 256;

template <int NT, int KPT = 8, int R = 1, typename ScoreAt, typename KeyAt>
__device__ void topk_select(ScoreAt score_at, KeyAt key_at, int c, int topk, int n_sink,
                            int n_local, int NA, int32_t* __restrict__ oidx,
                            float* __restrict__ osc, int* hist, int* sbuf, int* sh) {
  static_assert(NT >= 256 && NT % kWave == 0, "the select needs at least 256 threads");
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int n_sink_eff = min(n_sink, c + 1);
  const int lo = n_sink;                       // first candidate
  const int hi = c - n_local;                  // last candidate
  const int n = max(0, hi - lo + 1);
  const int K = min(topk, n);
  const int loc_beg = max(n_sink, c - n_local + 1);
  const int n_loc = max(0, c - loc_beg + 1);

  // forced entries and padding
  for (int i = tid; i < NA; i += NT) {
    if (i < n_sink_eff) {
      oidx[i] = i;
      osc[i] = score_at(i);
    } else if (i >= n_sink_eff + K) {
      const bool loc = i < n_sink_eff + K + n_loc;
      const int jj = loc_beg + (i - n_sink_eff - K);
      oidx[i] = loc ? jj : -1;
      osc[i] = loc ? score_at(jj) : 0.0f;
    }
  }
  if (K == 0) return;
  if (K == n) {
    for (int i = tid; i < n; i += NT) {
      oidx[n_sink_eff + i] = lo + i;
      osc[n_sink_eff + i] = score_at(lo + i);
    }
    return;
  }

  // each thread owns the contiguous slice beg..end of the candidates (index order for the
  // compaction); slices of at most KPT keys are held in registers for every pass
  const int per = (n + NT - 1) / NT;
  const int beg = min(n, tid * per);
  const int end = min(n, beg + per);
  const bool in_regs = per <= KPT;
  uint32_t kr[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) kr[j] = (in_regs && beg + j < end) ? key_at(beg + j) : 0u;

  // radix select of the K-th largest key, 8 bits at a time
  uint32_t prefix = 0u, mask = 0u;
  int krem = K;
  constexpr int HW = 256 * R;                  // words of one histogram
  for (int i = tid; i < HW; i += NT) hist[i] = 0;
  __syncthreads();
  const int rep = tid % R;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    int* h = hist + (pass & 1) * HW;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (beg + j < end && (kr[j] & mask) == prefix)
          atomicAdd(&h[((kr[j] >> shift) & 255u) * R + rep], 1);
    } else {
      for (int i = tid; i < n; i += NT) {     // strided: consecutive lanes, consecutive keys
        const uint32_t key = key_at(i);
        if ((key & mask) == prefix) atomicAdd(&h[((key >> shift) & 255u) * R + rep], 1);
      }
    }
    for (int i = tid; i < HW; i += NT) hist[((pass + 1) & 1) * HW + i] = 0;   // the next pass's
    __syncthreads();
    if (tid < kWave) {
      // lane l holds digits 255 - 4l .. 252 - 4l (descending)
      int c4[4], t4 = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c4[k] = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) c4[k] += h[(255 - 4 * lane - k) * R + r];
        t4 += c4[k];
      }
      const int incl = wave_inclusive_scan(t4);
      int above = incl - t4;                   // keys with larger digits than this lane's
      if (above < krem && krem <= incl) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (above < krem && krem <= above + c4[k]) {
            sh[0] = 255 - 4 * lane - k;
            sh[1] = krem - above;
          }
          above += c4[k];
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh[0] << shift;
    mask |= 255u << shift;
    krem = sh[1];
  }
  const uint32_t tau = prefix;
  const int need_eq = krem;                  // keys equal to tau to take, lowest index first

  // index-ordered compaction over the threads' slices
  int gt = 0, eq = 0;
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (beg + j < end) {
        gt += kr[j] > tau;
        eq += kr[j] == tau;
      }
  } else {
    for (int i = beg; i < end; ++i) {
      const uint32_t key = key_at(i);
      gt += key > tau;
      eq += key == tau;
    }
  }
  int tot, gt_before, eq_before;
  if (n < (1 << 15)) {
    const int packed = block_exclusive_scan<NT>(gt | (eq << 16), sbuf, &tot);
    gt_before = packed & 0xffff;
    eq_before = packed >> 16;
  } else {
    eq_before = block_exclusive_scan<NT>(eq, sbuf, &tot);
    gt_before = block_exclusive_scan<NT>(gt, sbuf, &tot);
  }
  const int take_eq = min(eq, max(0, need_eq - eq_before));
  int pos = gt_before + min(eq_before, need_eq);
  int eq_seen = 0;
  auto emit = [&](int i, uint32_t key) {
    bool take = key > tau;
    if (key == tau) {
      take = eq_seen < take_eq;
      ++eq_seen;
    }
    if (take) {
      oidx[n_sink_eff + pos] = lo + i;
      osc[n_sink_eff + pos] = score_at(lo + i);
      ++pos;
    }
  };
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (beg + j < end) emit(beg + j, kr[j]);
  } else {
    for (int i = beg; i < end; ++i) emit(i, key_at(i));
  }
}

}  // namespace bsa
