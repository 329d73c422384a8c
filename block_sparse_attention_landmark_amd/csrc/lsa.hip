// Flat clustered index over the landmarks (LSA page, "The index stops scanning the whole
// context", paragraphs 3-5): neighbouring keys are pooled first (the landmarks), Ward's algorithm
// groups similar landmarks of a completed segment into clusters, and the clustering is kept as
// each cluster's centre plus the table of its blocks; a query scores the centres (the flat
// variant scans them all), the best clusters are expanded back into blocks, and the start of the
// context and the recent window are added.
//
// lsa_ward_kernel    one workgroup per (sequence, kv group, completed segment of SEG <= 64
//                    landmarks): agglomerative Ward clustering down to NC clusters in LDS.  The
//                    merge cost of clusters A, B is |A||B| / (|A|+|B|) ||mean_A - mean_B||^2; the
//                    cheapest pair is merged (equal costs: the lexicographically smallest pair of
//                    ids, a cluster's id being its lowest member), and the merged cluster's costs
//                    are recomputed from its new mean.  Outputs: members (each cluster's blocks,
//                    ascending, clusters in id order), offsets, centres (the mean of the members'
//                    landmarks, float32) and the merge sequence.
// lsa_select_kernel  one workgroup per selection row: units = the clusters of the completed
//                    segments that lie wholly at or before the last candidate block, scored
//                    qbar . centre, and every other candidate block on its own, scored
//                    qbar . landmark; units sorted by (score descending, id ascending), expanded
//                    in that order into their candidate blocks until K are chosen (the last unit
//                    cut short); the row is the sink blocks, the chosen blocks ascending, the local
//                    window, then -1 padding; scores: a chosen block's unit score, else its own.
#include <math.h>
#include <stdint.h>

#include "bsa_common.hpp"
#include "bsa_internal.hpp"

namespace bsa {

constexpr int kLsaMaxSeg = 64;          // landmarks per segment held in LDS
constexpr int kLsaMaxUnits = 8192;      // units one selection row can sort
constexpr int kLsaMaxK = 2048;          // blocks one selection row can choose

// ---------------------------------------------------------------------------------------------
// Ward clustering of one segment
// ---------------------------------------------------------------------------------------------
template <int D, typename TIN>
__global__ __launch_bounds__(256) void lsa_ward_kernel(const TIN* __restrict__ lm,
                                                       float* __restrict__ centres,
                                                       int32_t* __restrict__ members,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ merges, int NB,
                                                       int NS, int SEG, int NC) {
  constexpr int MP = kLsaMaxSeg + 1;     // pitch of the transposed means: slot p of dim d at d*MP+p
  constexpr int S = kLsaMaxSeg;
  __shared__ float mt[D * MP];
  __shared__ float cost[S * S];
  __shared__ float sz[S];
  __shared__ int lab[S];
  __shared__ int alive[S];
  __shared__ int rank_[S];
  __shared__ int cnt[S + 1];
  __shared__ float rv[4];
  __shared__ int ri[4];
  __shared__ int pick[2];
  const int seg = blockIdx.x, bg = blockIdx.y;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int lo = seg * SEG;
  const TIN* L = lm + ((size_t)bg * NB + lo) * D;

  for (int e = tid; e < SEG * D; e += 256) {
    const int p = e / D, d = e % D;
    mt[d * MP + p] = (float)L[(size_t)p * D + d];
  }
  if (tid < S) {
    sz[tid] = 1.0f;
    lab[tid] = tid;
    alive[tid] = tid < SEG;
  }
  __syncthreads();
  // singleton costs: 1/2 ||x_i - x_j||^2 for i < j (a wave covers one row i)
  for (int e = tid; e < S * S; e += 256) {
    const int i = e / S, j = e % S;
    float cv = INFINITY;
    if (i < j && j < SEG) {
      float acc = 0.0f;
      for (int d = 0; d < D; ++d) {
        const float df = mt[d * MP + i] - mt[d * MP + j];
        acc = fmaf(df, df, acc);
      }
      cv = 0.5f * acc;
    }
    cost[e] = cv;
  }
  __syncthreads();

  int32_t* mrg = merges + ((size_t)bg * NS + seg) * (SEG - NC) * 2;
  for (int step = 0; step < SEG - NC; ++step) {
    // cheapest pair; equal costs: the smallest row-major position, i.e. the smallest (a, b)
    float best = INFINITY;
    int bi = S * S;
    for (int e = tid; e < S * S; e += 256) {
      const float cv = cost[e];
      if (cv < best) {
        best = cv;
        bi = e;
      }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov < best || (ov == best && oi < bi)) {
        best = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      rv[w] = best;
      ri[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float bb = rv[0];
      int ii = ri[0];
      for (int v = 1; v < 4; ++v)
        if (rv[v] < bb || (rv[v] == bb && ri[v] < ii)) {
          bb = rv[v];
          ii = ri[v];
        }
      pick[0] = ii / S;
      pick[1] = ii % S;
      mrg[2 * step] = lo + ii / S;
      mrg[2 * step + 1] = lo + ii % S;
    }
    __syncthreads();
    const int a = pick[0], b = pick[1];
    const float na = sz[a], nb = sz[b];
    for (int d = tid; d < D; d += 256) mt[d * MP + a] = (na * mt[d * MP + a] + nb * mt[d * MP + b]) / (na + nb);
    if (tid < S) {
      if (lab[tid] == b) lab[tid] = a;
      cost[b * S + tid] = INFINITY;
      cost[tid * S + b] = INFINITY;
    }
    __syncthreads();
    if (tid == 0) {
      sz[a] = na + nb;
      alive[b] = 0;
    }
    __syncthreads();
    // costs of the merged cluster against every other live one: 4 threads per cluster k
    {
      const int k = tid / 4, part = tid % 4;
      const bool live = k < SEG && alive[k] && k != a;
      float acc = 0.0f;
      if (live)
        for (int d = part; d < D; d += 4) {
          const float df = mt[d * MP + a] - mt[d * MP + k];
          acc = fmaf(df, df, acc);
        }
      acc += __shfl_xor(acc, 1, kWave);
      acc += __shfl_xor(acc, 2, kWave);
      if (live && part == 0) {
        const float sa = sz[a], sk = sz[k];
        cost[min(a, k) * S + max(a, k)] = sa * sk / (sa + sk) * acc;
      }
    }
    __syncthreads();
  }

  // clusters in id order: rank of each live slot; members grouped by cluster, ascending
  if (tid < S) rank_[tid] = 0;
  if (tid <= S) cnt[tid] = 0;
  __syncthreads();
  if (tid < SEG && alive[tid]) {
    int r = 0;
    for (int p = 0; p < tid; ++p) r += alive[p];
    rank_[tid] = r;
  }
  __syncthreads();
  if (tid < SEG) atomicAdd(&cnt[rank_[lab[tid]] + 1], 1);
  __syncthreads();
  if (tid == 0)
    for (int r = 0; r < NC; ++r) cnt[r + 1] += cnt[r];
  __syncthreads();
  const size_t sbase = (size_t)bg * NS + seg;
  if (tid < SEG) {
    const int r = rank_[lab[tid]];
    int before = 0;
    for (int p = 0; p < tid; ++p) before += lab[p] == lab[tid];
    members[sbase * SEG + cnt[r] + before] = lo + tid;
  }
  if (tid <= NC) offsets[sbase * (NC + 1) + tid] = cnt[tid];
  // centres: the mean of the members' landmarks, summed in ascending member order
  for (int e = tid; e < NC * D; e += 256) {
    const int r = e / D, d = e % D;
    float acc = 0.0f;
    int n = 0;
    for (int p = 0; p < SEG; ++p)
      if (rank_[lab[p]] == r) {
        acc += (float)L[(size_t)p * D + d];
        ++n;
      }
    centres[(sbase * NC + r) * D + d] = acc / (float)n;
  }
}

// ---------------------------------------------------------------------------------------------
// selection over the index
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void lsa_bitonic(uint64_t* key, int* pay, int m) {
  for (int k = 2; k <= m; k <<= 1)
    for (int s = k >> 1; s > 0; s >>= 1) {
      for (int i = threadIdx.x; i < m; i += blockDim.x) {
        const int p = i ^ s;
        if (p > i) {
          const bool up = (i & k) == 0;
          const uint64_t a = key[i], b = key[p];
          if ((a > b) == up) {
            key[i] = b;
            key[p] = a;
            const int t = pay[i];
            pay[i] = pay[p];
            pay[p] = t;
          }
        }
      }
      __syncthreads();
    }
}

// UCAP / KCAP: the units and chosen blocks one row can hold (LDS is sized by them, so a small
// variant lets several rows share a CU)
template <int D, typename TIN, int UCAP, int KCAP>
__global__ __launch_bounds__(256) void lsa_select_kernel(
    const float* __restrict__ qbar, const TIN* __restrict__ q, const TIN* __restrict__ lm,
    const float* __restrict__ centres, const int32_t* __restrict__ members,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ idx, float* __restrict__ sc, int Hq,
    int Hkv, int G, int NB, int NS, int SEG, int NC, int R, int c_dec, int topk, int n_sink,
    int n_local, int NA) {
  __shared__ float qv[D];
  // sort key: (order-preserving key of the score, inverted) << 32 | unit id; payload: unit index
  // | candidate blocks << 16 (a unit's score is recovered from its key)
  __shared__ uint64_t skey[UCAP];
  __shared__ int spay[UCAP];
  __shared__ int ch_blk[KCAP];
  __shared__ float ch_sc[KCAP];
  __shared__ int wsum[4];
  const int row = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int c = c_dec >= 0 ? c_dec : row;
  const TIN* Lg = lm + (size_t)bg * NB * D;

  // selector vector: prefill rows come precomputed; decode sums the group's query heads
  if (tid < D) {
    if (c_dec >= 0) {
      double acc = 0.0;
      for (int hh = 0; hh < G; ++hh) acc += (double)(float)q[(size_t)(b * Hq + g * G + hh) * D + tid];
      qv[tid] = (float)acc;
    } else {
      qv[tid] = qbar[((size_t)bg * R + row) * D + tid];
    }
  }
  __syncthreads();
  auto dot_lm = [&](int j) {
    float acc = 0.0f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) acc = fmaf(qv[d], (float)Lg[(size_t)j * D + d], acc);
    return acc;
  };

  const int last = c - n_local;
  const int n_elig = min(NS, max(0, (last + 1) / SEG));
  const int single_lo = max(n_sink, n_elig * SEG);
  const int n_single = max(0, last - single_lo + 1);
  const int n_units = n_elig * NC + n_single;
  int m = 1;
  while (m < n_units) m <<= 1;
  // unit u: a cluster (u < n_elig * NC) or the single block single_lo + u - n_elig * NC; its
  // score is a dot product over D spread on LPU lanes (8 elements each), UPW units per wave
  constexpr int LPU = D / 8;
  constexpr int UPW = kWave / LPU;
  const int sub = lane % LPU, uw = lane / LPU;
  float qf[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] = qv[sub * 8 + e];
  for (int u0 = w * UPW; u0 < m; u0 += 4 * UPW) {
    const int u = u0 + uw;
    float part = 0.0f;
    int size = 0;
    uint32_t id = 0;
    if (u < n_elig * NC) {
      const int sg = u / NC, r = u % NC;
      const size_t sb = (size_t)bg * NS + sg;
      const int o0 = offsets[sb * (NC + 1) + r], o1 = offsets[sb * (NC + 1) + r + 1];
      const int32_t* mem = members + sb * SEG;
      for (int i = o0; i < o1; ++i) size += mem[i] >= n_sink;
      id = (uint32_t)mem[o0];
      const f32x4* ctr = reinterpret_cast<const f32x4*>(centres + (sb * NC + r) * D + sub * 8);
      const f32x4 c0 = ctr[0], c1 = ctr[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) part = fmaf(qf[e], c0[e], fmaf(qf[4 + e], c1[e], part));
    } else if (u < n_units) {
      const int j = single_lo + (u - n_elig * NC);
      const TIN* lrow = Lg + (size_t)j * D + sub * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(qf[e], (float)lrow[e], part);
      size = 1;
      id = (uint32_t)j;
    }
#pragma unroll
    for (int o = LPU / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, kWave);
    if (sub == 0 && u < m) {
      uint64_t key = ~(uint64_t)0;
      if (u < n_units && size > 0) key = ((uint64_t)(~float_key(part)) << 32) | id;
      skey[u] = key;
      spay[u] = u | (size << 16);
    }
  }
  __syncthreads();
  lsa_bitonic(skey, spay, m);
  // blocks taken from each unit in sorted order: exclusive prefix of sizes, capped at K
  const int per = (m + 255) / 256;
  int local_sum = 0;
  for (int i = tid * per; i < min(m, (tid + 1) * per); ++i)
    if (skey[i] != ~(uint64_t)0) local_sum += spay[i] >> 16;
  int incl = local_sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wsum[w] = incl;
  __syncthreads();
  int base = incl - local_sum;
  for (int v = 0; v < w; ++v) base += wsum[v];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const int K = min(topk, total);
  for (int i = tid * per; i < min(m, (tid + 1) * per); ++i) {
    if (skey[i] == ~(uint64_t)0) continue;
    const int u = spay[i] & 0xffff;
    const int size = spay[i] >> 16;
    const float uscore = key_float(~(uint32_t)(skey[i] >> 32));
    if (base < K) {
      const int take = min(size, K - base);
      if (u < n_elig * NC) {
        const int sg = u / NC, r = u % NC;
        const size_t sb = (size_t)bg * NS + sg;
        const int o0 = offsets[sb * (NC + 1) + r], o1 = offsets[sb * (NC + 1) + r + 1];
        const int32_t* mem = members + sb * SEG;
        int n = 0;
        for (int x = o0; x < o1 && n < take; ++x)
          if (mem[x] >= n_sink) {
            ch_blk[base + n] = mem[x];
            ch_sc[base + n] = uscore;
            ++n;
          }
      } else {
        ch_blk[base] = single_lo + (u - n_elig * NC);
        ch_sc[base] = uscore;
      }
    }
    base += size;
  }
  __syncthreads();
  // chosen blocks ascending (the sort space is reused: block in the key, slot as payload)
  int mk = 1;
  while (mk < K) mk <<= 1;
  for (int i = tid; i < mk; i += 256) {
    skey[i] = i < K ? (uint64_t)(uint32_t)ch_blk[i] : ~(uint64_t)0;
    spay[i] = i;
  }
  __syncthreads();
  if (K > 1) lsa_bitonic(skey, spay, mk);
  // row: sink blocks, chosen blocks, local window, padding
  const int n_s = min(n_sink, c + 1);
  const int l0 = max(n_s, c - n_local + 1);      // local blocks that are not sink blocks
  const int n_l = max(0, c - l0 + 1);
  const size_t rb = ((size_t)bg * R + row) * NA;
  for (int i = tid; i < NA; i += 256) {
    int j = -1;
    float s = 0.0f;
    if (i < n_s) {
      j = i;
      s = dot_lm(j);
    } else if (i < n_s + K) {
      const int slot = spay[i - n_s];
      j = ch_blk[slot];
      s = ch_sc[slot];
    } else if (i < n_s + K + n_l) {
      j = l0 + (i - n_s - K);
      s = dot_lm(j);
    }
    idx[rb + i] = j;
    sc[rb + i] = s;
  }
}

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------
bool lsa_shape_ok(const Shape& s, int seg, int nc) {
  if (seg < 1 || seg > kLsaMaxSeg || nc < 1 || nc > seg) return false;
  const int ns = s.NB / seg;
  if ((int64_t)ns * nc + seg > kLsaMaxUnits) return false;
  return s.topk <= kLsaMaxK;
}

hipError_t launch_lsa_build(const Shape& s, const void* lm, int seg, int nc, float* centres,
                            int32_t* members, int32_t* offsets, int32_t* merges,
                            hipStream_t st) {
  const int ns = s.NB / seg;
  if (ns == 0) return hipSuccess;
  dim3 grid(ns, s.B * s.Hkv);
#define BSA_WARD(D_, T_)                                                                     \
  hipLaunchKernelGGL((lsa_ward_kernel<D_, T_>), grid, dim3(256), 0, st, (const T_*)lm, centres, \
                     members, offsets, merges, s.NB, ns, seg, nc)
  if (s.D == 128) {
    if (s.bf16) BSA_WARD(128, bf16);
    else BSA_WARD(128, float);
  } else {
    if (s.bf16) BSA_WARD(64, bf16);
    else BSA_WARD(64, float);
  }
#undef BSA_WARD
  return hipGetLastError();
}

hipError_t launch_lsa_select(const Shape& s, const void* q, const void* lm, int seg, int nc,
                             const float* centres, const int32_t* members,
                             const int32_t* offsets, int32_t* idx, float* sc, float* qbar,
                             hipStream_t st) {
  if (!s.decode) {
    const hipError_t e = launch_selector_vectors(s, q, qbar, st);
    if (e != hipSuccess) return e;
  }
  const int ns = s.NB / seg;
  dim3 grid(s.R, s.B * s.Hkv);
  const bool small = ns * nc + seg <= 1024 && s.topk <= 256;
#define BSA_LSEL(D_, T_, U_, K_)                                                                 \
  hipLaunchKernelGGL((lsa_select_kernel<D_, T_, U_, K_>), grid, dim3(256), 0, st, qbar,           \
                     (const T_*)q, (const T_*)lm, centres, members, offsets, idx, sc, s.Hq, s.Hkv, \
                     s.G, s.NB, ns, seg, nc, s.R, s.decode ? s.c_dec : -1, s.topk, s.n_sink,       \
                     s.n_local, s.NA)
#define BSA_LSEL_CAP(D_, T_)                          \
  if (small) BSA_LSEL(D_, T_, 1024, 256);             \
  else BSA_LSEL(D_, T_, kLsaMaxUnits, kLsaMaxK);
  if (s.D == 128) {
    if (s.bf16) {
      BSA_LSEL_CAP(128, bf16)
    } else {
      BSA_LSEL_CAP(128, float)
    }
  } else {
    if (s.bf16) {
      BSA_LSEL_CAP(64, bf16)
    } else {
      BSA_LSEL_CAP(64, float)
    }
  }
#undef BSA_LSEL_CAP
#undef BSA_LSEL
  return hipGetLastError();
}

}  // namespace bsa
