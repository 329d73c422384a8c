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

#include <algorithm>

#include "bsa_common.hpp"
#include "bsa_internal.hpp"
#include "select_common.hpp"

namespace bsa {

constexpr int kLsaMaxSeg = 64;          // landmarks per segment held in LDS
constexpr int kLsaMaxUnits = 8192;      // units one selection row can sort
constexpr int kLsaMaxK = 2048;          // blocks one selection row can choose
constexpr size_t kLsaScoreBuf = 256u << 20;  // bytes of precomputed cluster scores per call

// ---------------------------------------------------------------------------------------------
// Ward clustering of one segment
// ---------------------------------------------------------------------------------------------
template <int D, typename TIN>
__global__ __launch_bounds__(256) void lsa_ward_kernel(const TIN* __restrict__ lm,
                                                       float* __restrict__ centres,
                                                       int32_t* __restrict__ members,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ merges, int NB,
                                                       int NS, int SEG, int NC, int seg0) {
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
  const int seg = seg0 + blockIdx.x, bg = blockIdx.y;
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
// variant lets several rows share a CU).  The units are laid out in id order (the clusters of
// each segment by id, segments ascending, then the single blocks ascending), so the shared radix
// top-K -- which takes the lower index first among equal scores -- ranks them by (score
// descending, id ascending); only the min(K, units) best units are then sorted, since every unit
// with a candidate block contributes at least one block.
//
// PRE: the cluster scores of rows row0 .. row0 + gridDim.x - 1 were formed beforehand by
// lsa_unit_scores_kernel (upre, nrows x NS*NC per (sequence, kv group)) and the clusters'
// candidate counts by lsa_unit_sizes_kernel (usizes); the single blocks are still scored here.
template <int D, typename TIN, int UCAP, int KCAP, bool PRE>
__global__ __launch_bounds__(256) void lsa_select_kernel(
    const float* __restrict__ qbar, const TIN* __restrict__ q, const TIN* __restrict__ lm,
    const float* __restrict__ centres, const int32_t* __restrict__ members,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ idx, float* __restrict__ sc, int Hq,
    int Hkv, int G, int NB, int NS, int SEG, int NC, int R, int c_dec, int topk, int n_sink,
    int n_local, int NA, const float* __restrict__ upre, const uint16_t* __restrict__ usizes,
    int row0, int nrows) {
  __shared__ float qv[D];
  __shared__ float uscore[UCAP];     // unit score; -inf for a unit without candidate blocks
  __shared__ uint16_t usize[UCAP];   // candidate blocks of the unit (at most kLsaMaxSeg)
  __shared__ int32_t tsel[KCAP + 1]; // the best units (ascending unit index), then a dummy entry
  __shared__ float tsc[KCAP + 1];
  // sort space: (order-preserving key of the score, inverted) << 32 | unit index, payload = the
  // unit; reused for the chosen blocks
  __shared__ uint64_t skey[KCAP];
  __shared__ int spay[KCAP];
  __shared__ int ch_blk[KCAP];
  __shared__ float ch_sc[KCAP];
  __shared__ int hist[kTopkHistWords];
  __shared__ int sbuf[4];
  __shared__ int sh[2];
  __shared__ int wsum[4];
  const int row = row0 + (int)blockIdx.x, bg = blockIdx.y;
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
  // unit u: a cluster (u < n_elig * NC) or the single block single_lo + u - n_elig * NC; its
  // score is a dot product over D spread on LPU lanes (8 elements each), UPW units per wave
  constexpr int LPU = D / 8;
  constexpr int UPW = kWave / LPU;
  const int sub = lane % LPU, uw = lane / LPU;
  float qf[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] = qv[sub * 8 + e];
  int u_first = 0;                                 // first unit scored by the loop below
  if constexpr (PRE) {
    const float* urow = upre + ((size_t)bg * nrows + (row - row0)) * (size_t)(NS * NC);
    const uint16_t* usz = usizes + (size_t)bg * NS * NC;
    for (int u = tid; u < n_elig * NC; u += 256) {
      const int size = usz[u];
      uscore[u] = size > 0 ? urow[u] : -INFINITY;
      usize[u] = (uint16_t)size;
    }
    u_first = n_elig * NC;
  }
  // UB units per lane group in flight (their loads issued together)
  constexpr int UB = 4;
  for (int u0 = u_first + w * UPW; u0 < n_units; u0 += 4 * UPW * UB) {
    float part[UB];
    int size[UB];
#pragma unroll
    for (int k = 0; k < UB; ++k) {
      const int u = u0 + uw + k * 4 * UPW;
      part[k] = 0.0f;
      size[k] = 0;
      if (u < n_elig * NC) {
        const int sg = u / NC, r = u % NC;
        const size_t sb = (size_t)bg * NS + sg;
        const int o0 = offsets[sb * (NC + 1) + r], o1 = offsets[sb * (NC + 1) + r + 1];
        if (sg * SEG < n_sink) {                // a segment holding sink blocks: count members
          const int32_t* mem = members + sb * SEG;
          for (int i = o0; i < o1; ++i) size[k] += mem[i] >= n_sink;
        } else {
          size[k] = o1 - o0;                    // every member is a candidate
        }
        const f32x4* ctr = reinterpret_cast<const f32x4*>(centres + (sb * NC + r) * D + sub * 8);
        const f32x4 c0 = ctr[0], c1 = ctr[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) part[k] = fmaf(qf[e], c0[e], fmaf(qf[4 + e], c1[e], part[k]));
      } else if (u < n_units) {
        const int j = single_lo + (u - n_elig * NC);
        const TIN* lrow = Lg + (size_t)j * D + sub * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) part[k] = fmaf(qf[e], (float)lrow[e], part[k]);
        size[k] = 1;
      }
    }
#pragma unroll
    for (int k = 0; k < UB; ++k) {
      const int u = u0 + uw + k * 4 * UPW;
#pragma unroll
      for (int o = LPU / 2; o > 0; o >>= 1) part[k] += __shfl_xor(part[k], o, kWave);
      if (sub == 0 && u < n_units) {
        uscore[u] = size[k] > 0 ? part[k] : -INFINITY;
        usize[u] = (uint16_t)size[k];
      }
    }
  }
  __syncthreads();
  // the best min(topk, units) units, ascending unit index (ties: the lower index)
  const int KU = min(topk, n_units);
  topk_select<256>([&](int u) { return u < n_units ? uscore[u] : 0.0f; },
                   [&](int i) { return float_key(uscore[i]); }, n_units, KU, 0, 1, KU + 1, tsel,
                   tsc, hist, sbuf, sh);
  __syncthreads();
  // those units in selection order: score descending, unit index ascending
  int m = 1;
  while (m < KU) m <<= 1;
  for (int i = tid; i < m; i += 256) {
    uint64_t key = ~(uint64_t)0;
    int u = 0;
    if (i < KU) {
      u = tsel[i];
      key = ((uint64_t)(~float_key(uscore[u])) << 32) | (uint32_t)u;
    }
    skey[i] = key;
    spay[i] = u;
  }
  __syncthreads();
  if (KU > 1) lsa_bitonic(skey, spay, m);
  // blocks taken from each unit in sorted order: exclusive prefix of sizes, capped at K
  const int per = (m + 255) / 256;
  int local_sum = 0;
  for (int i = tid * per; i < min(KU, (tid + 1) * per); ++i) local_sum += usize[spay[i]];
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
  for (int i = tid * per; i < min(KU, (tid + 1) * per); ++i) {
    const int u = spay[i];
    const int size = usize[u];
    const float us = uscore[u];
    if (base < K && size > 0) {
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
            ch_sc[base + n] = us;
            ++n;
          }
      } else {
        ch_blk[base] = single_lo + (u - n_elig * NC);
        ch_sc[base] = us;
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
// tree index: node centres, beam-search selection
// ---------------------------------------------------------------------------------------------
// Above the Ward clusters of a segment sits the segment, above segments groups of FAN
// consecutive segments; a node's centre is the mean of the landmarks under it (LSA page, the
// same section, paragraph 5: the tree variant joins clusters into a hierarchy and walks it by
// beam search, keeping a few branches per level).

// one workgroup per (segment, sequence x kv group): the segment's centre; segments that close a
// group of FAN also write the group's centre (the mean of its segments' centres)
template <int D, typename TIN>
__global__ __launch_bounds__(128) void lsa_tree_centres_kernel(const TIN* __restrict__ lm,
                                                               float* __restrict__ seg_c,
                                                               float* __restrict__ grp_c, int NB,
                                                               int NS, int NG, int SEG, int FAN) {
  const int s = blockIdx.x, bg = blockIdx.y;
  for (int d = threadIdx.x; d < D; d += 128) {
    const TIN* L = lm + ((size_t)bg * NB + (size_t)s * SEG) * D + d;
    float acc = 0.0f;
    for (int p = 0; p < SEG; ++p) acc += (float)L[(size_t)p * D];
    seg_c[((size_t)bg * NS + s) * D + d] = acc / (float)SEG;
  }
  if ((s + 1) % FAN != 0 || (s + 1) / FAN > NG) return;
  const int gi = s / FAN;
  // the group's centre is formed by the segment that closes it from the landmarks directly (the
  // other segments' centres may not be written yet): mean over FAN * SEG landmarks
  for (int d = threadIdx.x; d < D; d += 128) {
    float acc = 0.0f;
    for (int t = 0; t < FAN; ++t) {
      const TIN* L = lm + ((size_t)bg * NB + (size_t)(gi * FAN + t) * SEG) * D + d;
      float a2 = 0.0f;
      for (int p = 0; p < SEG; ++p) a2 += (float)L[(size_t)p * D];
      acc += a2 / (float)SEG;
    }
    grp_c[((size_t)bg * NG + gi) * D + d] = acc / (float)FAN;
  }
}

template <int D, typename TIN, int KCAP>
__global__ __launch_bounds__(256) void lsa_tree_select_kernel(
    const float* __restrict__ qbar, const TIN* __restrict__ q, const TIN* __restrict__ lm,
    const float* __restrict__ centres, const int32_t* __restrict__ members,
    const int32_t* __restrict__ offsets, const float* __restrict__ seg_c,
    const float* __restrict__ grp_c, int32_t* __restrict__ idx, float* __restrict__ sc, int Hq,
    int Hkv, int G, int NB, int NS, int NG, int SEG, int NC, int FAN, int BEAM, int R, int c_dec,
    int topk, int n_sink, int n_local, int NA) {
  constexpr int CAP = 1024;
  __shared__ float qv[D];
  __shared__ uint64_t skey[CAP];
  __shared__ int spay[CAP];
  __shared__ int cand[CAP];                      // candidate node ids of the next level
  __shared__ int kept[64];
  __shared__ int ch_blk[KCAP];
  __shared__ float ch_sc[KCAP];
  __shared__ int wsum[4];
  __shared__ int ncand_s;
  const int row = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int c = c_dec >= 0 ? c_dec : row;
  const TIN* Lg = lm + (size_t)bg * NB * D;
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
  constexpr int LPU = D / 8;
  constexpr int UPW = kWave / LPU;
  const int sub = lane % LPU, uw = lane / LPU;
  float qf[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] = qv[sub * 8 + e];
  // Score n nodes: node u's centre row is ctr(u) (float32), its id (first block) id(u), its
  // candidate size size(u) (0: not a unit); sort them by (score desc, id asc).  Returns the
  // sort length.
  auto score_sort = [&](int n, auto ctr, auto id_of, auto size_of) {
    int m = 1;
    while (m < n) m <<= 1;
    for (int u0 = w * UPW; u0 < m; u0 += 4 * UPW) {
      const int u = u0 + uw;
      float part = 0.0f;
      if (u < n) {
        const f32x4* cp = reinterpret_cast<const f32x4*>(ctr(u) + sub * 8);
        const f32x4 c0 = cp[0], c1 = cp[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fmaf(qf[e], c0[e], fmaf(qf[4 + e], c1[e], part));
      }
#pragma unroll
      for (int o = LPU / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, kWave);
      if (sub == 0 && u < m) {
        uint64_t key = ~(uint64_t)0;
        int size = 0;
        if (u < n) {
          size = size_of(u);
          if (size > 0) key = ((uint64_t)(~float_key(part)) << 32) | (uint32_t)id_of(u);
        }
        skey[u] = key;
        spay[u] = u | (size << 16);
      }
    }
    __syncthreads();
    lsa_bitonic(skey, spay, m);
    return m;
  };

  const int last = c - n_local;
  const int n_elig = min(NS, max(0, (last + 1) / SEG));
  const int n_grp = min(NG, n_elig / FAN);
  const int n_left = n_elig - n_grp * FAN;
  // level 1: whole groups, and the eligible segments not in a whole group
  {
    const int n = n_grp + n_left;
    score_sort(n,
               [&](int u) { return u < n_grp ? grp_c + ((size_t)bg * NG + u) * D
                                             : seg_c + ((size_t)bg * NS + n_grp * FAN + (u - n_grp)) * D; },
               [&](int u) { return u < n_grp ? u * FAN * SEG : (n_grp * FAN + (u - n_grp)) * SEG; },
               [&](int) { return 1; });
    // candidate segments of the kept nodes
    if (tid == 0) {
      int nc = 0;
      for (int i = 0; i < min(BEAM, n); ++i) {
        const int u = spay[i] & 0xffff;
        if (u < n_grp)
          for (int t = 0; t < FAN; ++t) cand[nc++] = u * FAN + t;
        else
          cand[nc++] = n_grp * FAN + (u - n_grp);
      }
      ncand_s = nc;
    }
    __syncthreads();
  }
  // level 2: segments
  {
    const int n = ncand_s;
    score_sort(n, [&](int u) { return seg_c + ((size_t)bg * NS + cand[u]) * D; },
               [&](int u) { return cand[u] * SEG; }, [&](int) { return 1; });
    if (tid < min(BEAM, n)) kept[tid] = cand[spay[tid] & 0xffff];
    if (tid == 0) ncand_s = min(BEAM, n);
    __syncthreads();
  }
  // level 3: the clusters of the kept segments
  const int nseg = ncand_s;
  {
    const int n = nseg * NC;
    auto cl_off = [&](int u, int k) {
      const size_t sb = (size_t)bg * NS + kept[u / NC];
      return offsets[sb * (NC + 1) + u % NC + k];
    };
    score_sort(n, [&](int u) { return centres + (((size_t)bg * NS + kept[u / NC]) * NC + u % NC) * D; },
               [&](int u) { return members[((size_t)bg * NS + kept[u / NC]) * SEG + cl_off(u, 0)]; },
               [&](int u) {
                 const int32_t* mem = members + ((size_t)bg * NS + kept[u / NC]) * SEG;
                 int sz = 0;
                 for (int i = cl_off(u, 0); i < cl_off(u, 1); ++i) sz += mem[i] >= n_sink;
                 return sz;
               });
    // kept clusters become units: cand[i] = cluster u (segment slot u / NC, cluster u % NC)
    if (tid == 0) {
      int nc = 0;
      for (int i = 0; i < min(BEAM, n); ++i)
        if (skey[i] != ~(uint64_t)0) cand[nc++] = spay[i] & 0xffff;
      ncand_s = nc;
    }
    __syncthreads();
  }
  // units: the kept clusters and the not yet clustered candidate blocks, expanded to K blocks
  const int n_cl = ncand_s;
  const int single_lo = max(n_sink, n_elig * SEG);
  const int n_single = max(0, last - single_lo + 1);
  const int n_units = n_cl + n_single;
  auto unit_members = [&](int u, int& o0, int& o1) -> const int32_t* {
    const int cu = cand[u];
    const size_t sb = (size_t)bg * NS + kept[cu / NC];
    o0 = offsets[sb * (NC + 1) + cu % NC];
    o1 = offsets[sb * (NC + 1) + cu % NC + 1];
    return members + sb * SEG;
  };
  int m = 1;
  while (m < n_units) m <<= 1;
  for (int u0 = w * UPW; u0 < m; u0 += 4 * UPW) {
    const int u = u0 + uw;
    float part = 0.0f;
    int size = 0;
    uint32_t id = 0;
    if (u < n_cl) {
      int o0, o1;
      const int32_t* mem = unit_members(u, o0, o1);
      for (int i = o0; i < o1; ++i) size += mem[i] >= n_sink;
      id = (uint32_t)mem[o0];
      const int cu = cand[u];
      const f32x4* cp = reinterpret_cast<const f32x4*>(
          centres + (((size_t)bg * NS + kept[cu / NC]) * NC + cu % NC) * D + sub * 8);
      const f32x4 c0 = cp[0], c1 = cp[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) part = fmaf(qf[e], c0[e], fmaf(qf[4 + e], c1[e], part));
    } else if (u < n_units) {
      const int j = single_lo + (u - n_cl);
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
      if (u < n_cl) {
        int o0, o1;
        const int32_t* mem = unit_members(u, o0, o1);
        int n = 0;
        for (int x = o0; x < o1 && n < take; ++x)
          if (mem[x] >= n_sink) {
            ch_blk[base + n] = mem[x];
            ch_sc[base + n] = uscore;
            ++n;
          }
      } else {
        ch_blk[base] = single_lo + (u - n_cl);
        ch_sc[base] = uscore;
      }
    }
    base += size;
  }
  __syncthreads();
  int mk = 1;
  while (mk < K) mk <<= 1;
  for (int i = tid; i < mk; i += 256) {
    skey[i] = i < K ? (uint64_t)(uint32_t)ch_blk[i] : ~(uint64_t)0;
    spay[i] = i;
  }
  __syncthreads();
  if (K > 1) lsa_bitonic(skey, spay, mk);
  const int n_s = min(n_sink, c + 1);
  const int l0 = max(n_s, c - n_local + 1);
  const int n_l = max(0, c - l0 + 1);
  const size_t rb = ((size_t)bg * R + row) * NA;
  auto dot_lm = [&](int j) {
    float acc = 0.0f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) acc = fmaf(qv[d], (float)Lg[(size_t)j * D + d], acc);
    return acc;
  };
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
// beam search with one wave per prefill selection row
// ---------------------------------------------------------------------------------------------
// The per-row work of lsa_tree_select_kernel is a few hundred short dot products and five sorts
// of at most a few hundred keys: a latency-bound chain of loads.  Here each wave owns one row
// (four rows per workgroup, no barrier at all, eight waves per SIMD): each level's nodes are
// sorted in the wave's registers (element e = 64 s + lane, lane exchanges by shuffles), node
// loads are batched, a cluster's candidate count comes from its offsets unless its segment holds
// sink blocks, a chosen cluster is expanded by the whole wave, and landmark rows are read 16
// bytes at a time.  Scores (the same lanes per node, the same multiply-add order and shuffle
// tree), keys, tie rule and expansion are those of lsa_tree_select_kernel, so both give the same
// rows bit for bit.

// makes a wave's LDS writes visible to its other lanes before they read them
__device__ __forceinline__ void lsa_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// one wave sorts key[0..m) ascending with its payload, m a power of two <= 256
__device__ __forceinline__ void lsa_bitonic_wave(uint64_t* key, int* pay, int m) {
  const int lane = threadIdx.x % kWave;
  const int nreg = m > kWave ? m / kWave : 1;
  uint64_t kv[4];
  int pv[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = s * kWave + lane;
    const bool in = s < nreg && e < m;
    kv[s] = in ? key[e] : ~(uint64_t)0;
    pv[s] = in ? pay[e] : 0;
  }
  for (int k = 2; k <= m; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kWave) {                            // partner in another register of this lane
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int t = s ^ (j / kWave);
          if (t > s && t < nreg) {
            const bool up = ((s * kWave + lane) & k) == 0;
            if ((kv[s] > kv[t]) == up) {
              const uint64_t a = kv[s];
              kv[s] = kv[t];
              kv[t] = a;
              const int b = pv[s];
              pv[s] = pv[t];
              pv[t] = b;
            }
          }
        }
      } else {                                     // partner in lane ^ j, same register
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s < nreg) {
            const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)kv[s], j, kWave);
            const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(kv[s] >> 32), j, kWave);
            const int op = __shfl_xor(pv[s], j, kWave);
            const uint64_t o = ((uint64_t)hi << 32) | lo;
            const bool up = ((s * kWave + lane) & k) == 0;
            const bool lower = (lane & j) == 0;
            if (lower == up ? o < kv[s] : o > kv[s]) {
              kv[s] = o;
              pv[s] = op;
            }
          }
        }
      }
    }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = s * kWave + lane;
    if (s < nreg && e < m) {
      key[e] = kv[s];
      pay[e] = pv[s];
    }
  }
}

constexpr int kTreeWaveCap = 256;                  // nodes of one level, units, chosen blocks

// CAP (128 or 256) bounds a level's nodes, the units and the chosen blocks of a row; LDS is sized
// by it, so the smaller variant holds more rows per CU.  The row chain is latency-bound, so the
// register budget is held to eight waves per SIMD (a few registers spill; 20 % faster at 1M
// tokens than four waves per SIMD without spills).
//
// FUSEQ (bf16): the wave forms its row's selector vector from Q itself -- the sum over the
// group's heads of the mean over the block's tokens, summed in float64 and rounded once to
// float32, as the selector-vector pass does (the float64 sums of bf16 values are exact unless
// their magnitudes span more than about 2^40, so the different summation order gives the same
// vector) -- and Q is read while other rows search the tree.
template <int D, typename TIN, int CAP, bool FUSEQ>
__global__ __launch_bounds__(256, CAP == 128 ? 8 : 4) void lsa_tree_select_wave_kernel(
    const float* __restrict__ qbar, const TIN* __restrict__ q, const TIN* __restrict__ lm,
    const float* __restrict__ centres, const int32_t* __restrict__ members,
    const int32_t* __restrict__ offsets, const float* __restrict__ seg_c,
    const float* __restrict__ grp_c, int32_t* __restrict__ idx, float* __restrict__ sc, int Hq,
    int Hkv, int G, int T, int NB, int NS, int NG, int SEG, int NC, int FAN, int BEAM, int R,
    int topk, int n_sink, int n_local, int NA) {
  static_assert(CAP <= kTreeWaveCap && CAP / 2 >= 64, "sort width and chosen-cluster slots");
  __shared__ float qv_s[4][D];
  __shared__ uint64_t skey_s[4][CAP];
  __shared__ int spay_s[4][CAP];
  __shared__ int cand_s[4][CAP];
  __shared__ int kept_s[4][64];
  __shared__ int ch_blk_s[4][CAP];
  __shared__ float ch_sc_s[4][CAP];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int row = blockIdx.x * 4 + w;
  const int bg = blockIdx.y;
  if (row >= R) return;                            // no barrier follows: the wave may leave
  float* qv = qv_s[w];
  uint64_t* skey = skey_s[w];
  int* spay = spay_s[w];
  int* cand = cand_s[w];
  int* kept = kept_s[w];
  int* ch_blk = ch_blk_s[w];
  float* ch_sc = ch_sc_s[w];
  const int c = row;
  const TIN* Lg = lm + (size_t)bg * NB * D;
  if constexpr (FUSEQ) {
    constexpr int NCH = D / 8;                     // 16-byte chunks of a row
    constexpr int RGW = kWave / NCH;               // (head, token) rows in flight per load
    constexpr int NL = 8;                          // loads in flight per lane
    const int chunk = lane % NCH, rg = lane / NCH;
    const int b = bg / Hkv, g = bg % Hkv;
    const int t0 = c * kBlock, ntok = min(kBlock, T - t0);
    const int nr = G * ntok;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int r0 = rg; r0 < nr; r0 += RGW * NL) {
      u32x4 raw[NL];
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        const int rr = min(r0 + k * RGW, nr - 1);
        const int hh = rr / ntok, t = t0 + rr % ntok;
        raw[k] = *reinterpret_cast<const u32x4*>(q + ((size_t)(b * Hq + g * G + hh) * T + t) * D +
                                                 chunk * 8);
      }
#pragma unroll
      for (int k = 0; k < NL; ++k)
        if (r0 + k * RGW < nr) {
          const bf16x8 x = __builtin_bit_cast(bf16x8, raw[k]);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += (double)bf2f(x[e]);
        }
    }
#pragma unroll
    for (int o = NCH; o < kWave; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
    if (rg == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[chunk * 8 + e] = (float)(acc[e] / (double)ntok);
  } else {
    for (int d = lane; d < D; d += kWave) qv[d] = qbar[((size_t)bg * R + row) * D + d];
  }
  lsa_wave_sync();
  constexpr int LPU = D / 8;
  constexpr int UPW = kWave / LPU;
  constexpr int UB = 4;
  const int sub = lane % LPU, uw = lane / LPU;
  float qf[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] = qv[sub * 8 + e];
  // Score n nodes (centre row ctr(u), id id_of(u), candidate size size_of(u), 0: not a unit) and
  // sort them by (score desc, id asc); returns the sort length
  auto score_sort = [&](int n, auto ctr, auto id_of, auto size_of) {
    int m = 1;
    while (m < n) m <<= 1;
    for (int u0 = 0; u0 < m; u0 += UPW * UB) {    // UB nodes per lane group in flight
      float part[UB];
#pragma unroll
      for (int t = 0; t < UB; ++t) {
        const int u = u0 + uw + t * UPW;
        part[t] = 0.0f;
        if (u < n) {
          const f32x4* cp = reinterpret_cast<const f32x4*>(ctr(u) + sub * 8);
          const f32x4 c0 = cp[0], c1 = cp[1];
#pragma unroll
          for (int e = 0; e < 4; ++e) part[t] = fmaf(qf[e], c0[e], fmaf(qf[4 + e], c1[e], part[t]));
        }
      }
#pragma unroll
      for (int t = 0; t < UB; ++t) {
        const int u = u0 + uw + t * UPW;
#pragma unroll
        for (int o = LPU / 2; o > 0; o >>= 1) part[t] += __shfl_xor(part[t], o, kWave);
        if (sub == 0 && u < m) {
          uint64_t key = ~(uint64_t)0;
          int size = 0;
          if (u < n) {
            size = size_of(u);
            if (size > 0) key = ((uint64_t)(~float_key(part[t])) << 32) | (uint32_t)id_of(u);
          }
          skey[u] = key;
          spay[u] = u | (size << 16);
        }
      }
    }
    lsa_wave_sync();
    lsa_bitonic_wave(skey, spay, m);
    lsa_wave_sync();
    return m;
  };

  const int last = c - n_local;
  const int n_elig = min(NS, max(0, (last + 1) / SEG));
  const int n_grp = min(NG, n_elig / FAN);
  const int n_left = n_elig - n_grp * FAN;
  // level 1: whole groups, and the eligible segments not in a whole group
  int ncand;
  {
    const int n = n_grp + n_left;
    score_sort(n,
               [&](int u) { return u < n_grp ? grp_c + ((size_t)bg * NG + u) * D
                                             : seg_c + ((size_t)bg * NS + n_grp * FAN + (u - n_grp)) * D; },
               [&](int u) { return u < n_grp ? u * FAN * SEG : (n_grp * FAN + (u - n_grp)) * SEG; },
               [&](int) { return 1; });
    // candidate segments of the kept nodes: lane i < beam writes its node's children at the
    // exclusive prefix of the child counts
    const int nk = min(BEAM, n);
    int u = 0, cnt = 0;
    if (lane < nk) {
      u = spay[lane] & 0xffff;
      cnt = u < n_grp ? FAN : 1;
    }
    const int incl = wave_inclusive_scan(cnt);
    ncand = __shfl(incl, kWave - 1, kWave);
    if (lane < nk) {
      const int o = incl - cnt;
      if (u < n_grp)
        for (int t = 0; t < FAN; ++t) cand[o + t] = u * FAN + t;
      else
        cand[o] = n_grp * FAN + (u - n_grp);
    }
    lsa_wave_sync();
  }
  // level 2: segments
  int nseg;
  {
    const int n = ncand;
    score_sort(n, [&](int u) { return seg_c + ((size_t)bg * NS + cand[u]) * D; },
               [&](int u) { return cand[u] * SEG; }, [&](int) { return 1; });
    nseg = min(BEAM, n);
    if (lane < nseg) kept[lane] = cand[spay[lane] & 0xffff];
    lsa_wave_sync();
  }
  // level 3: the clusters of the kept segments; the kept clusters become units
  int n_cl;
  {
    const int n = nseg * NC;
    auto cl_off = [&](int u, int k) {
      const size_t sb = (size_t)bg * NS + kept[u / NC];
      return offsets[sb * (NC + 1) + u % NC + k];
    };
    score_sort(n, [&](int u) { return centres + (((size_t)bg * NS + kept[u / NC]) * NC + u % NC) * D; },
               [&](int u) { return members[((size_t)bg * NS + kept[u / NC]) * SEG + cl_off(u, 0)]; },
               [&](int u) {
                 const int o0 = cl_off(u, 0), o1 = cl_off(u, 1);
                 if (kept[u / NC] * SEG >= n_sink) return o1 - o0;   // no sink block here
                 const int32_t* mem = members + ((size_t)bg * NS + kept[u / NC]) * SEG;
                 int sz = 0;
                 for (int i = o0; i < o1; ++i) sz += mem[i] >= n_sink;
                 return sz;
               });
    const int nk = min(BEAM, n);
    const bool live = lane < nk && skey[lane] != ~(uint64_t)0;
    const uint64_t lm_ = __ballot(live);
    const int o = __popcll(lm_ & ((1ull << lane) - 1ull));
    if (live) cand[o] = spay[lane] & 0xffff;
    n_cl = __popcll(lm_);
    lsa_wave_sync();
  }
  // units: the kept clusters (cand[u] = segment slot * NC + cluster) and the not yet clustered
  // candidate blocks, sorted by (score desc, id asc) and expanded to K blocks
  const int single_lo = max(n_sink, n_elig * SEG);
  const int n_single = max(0, last - single_lo + 1);
  const int n_units = n_cl + n_single;
  auto unit_members = [&](int u, int& o0, int& o1) -> const int32_t* {
    const int cu = cand[u];
    const size_t sb = (size_t)bg * NS + kept[cu / NC];
    o0 = offsets[sb * (NC + 1) + cu % NC];
    o1 = offsets[sb * (NC + 1) + cu % NC + 1];
    return members + sb * SEG;
  };
  int m = 1;
  while (m < n_units) m <<= 1;
  for (int u0 = 0; u0 < m; u0 += UPW * UB) {
    float part[UB];
    int size[UB];
    uint32_t id[UB];
#pragma unroll
    for (int t = 0; t < UB; ++t) {
      const int u = u0 + uw + t * UPW;
      part[t] = 0.0f;
      size[t] = 0;
      id[t] = 0;
      if (u < n_cl) {
        int o0, o1;
        const int32_t* mem = unit_members(u, o0, o1);
        if (kept[cand[u] / NC] * SEG >= n_sink) {
          size[t] = o1 - o0;
        } else {
          for (int i = o0; i < o1; ++i) size[t] += mem[i] >= n_sink;
        }
        id[t] = (uint32_t)mem[o0];
        const int cu = cand[u];
        const f32x4* cp = reinterpret_cast<const f32x4*>(
            centres + (((size_t)bg * NS + kept[cu / NC]) * NC + cu % NC) * D + sub * 8);
        const f32x4 c0 = cp[0], c1 = cp[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) part[t] = fmaf(qf[e], c0[e], fmaf(qf[4 + e], c1[e], part[t]));
      } else if (u < n_units) {
        const int j = single_lo + (u - n_cl);
        const TIN* lrow = Lg + (size_t)j * D + sub * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) part[t] = fmaf(qf[e], (float)lrow[e], part[t]);
        size[t] = 1;
        id[t] = (uint32_t)j;
      }
    }
#pragma unroll
    for (int t = 0; t < UB; ++t) {
      const int u = u0 + uw + t * UPW;
#pragma unroll
      for (int o = LPU / 2; o > 0; o >>= 1) part[t] += __shfl_xor(part[t], o, kWave);
      if (sub == 0 && u < m) {
        uint64_t key = ~(uint64_t)0;
        if (u < n_units && size[t] > 0) key = ((uint64_t)(~float_key(part[t])) << 32) | id[t];
        skey[u] = key;
        spay[u] = u | (size[t] << 16);
      }
    }
  }
  lsa_wave_sync();
  lsa_bitonic_wave(skey, spay, m);
  lsa_wave_sync();
  // blocks taken from each unit in sorted order: lane l holds sorted entries 4l .. 4l+3
  int sz4[4], local_sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * lane + k;
    sz4[k] = (i < m && skey[i] != ~(uint64_t)0) ? (spay[i] >> 16) : 0;
    local_sum += sz4[k];
  }
  const int incl = wave_inclusive_scan(local_sum);
  const int total = __shfl(incl, kWave - 1, kWave);
  const int K = min(topk, total);
  int base = incl - local_sum;
  // single blocks are written by the lanes that hold them; the chosen clusters (at most beam) are
  // collected and then expanded by the whole wave, one member per lane
  int n_take = 0;                                  // chosen clusters so far (wave-uniform)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * lane + k;
    const bool chosen = sz4[k] > 0 && base < K;
    const int u = chosen ? (spay[i] & 0xffff) : 0;
    const bool is_cl = chosen && u < n_cl;
    if (chosen && !is_cl) {
      ch_blk[base] = single_lo + (u - n_cl);
      ch_sc[base] = key_float(~(uint32_t)(skey[i] >> 32));
    }
    const uint64_t bm = __ballot(is_cl);
    if (is_cl) {                                  // slot in the wave's list of chosen clusters
      const int t = n_take + __popcll(bm & ((1ull << lane) - 1ull));
      cand[CAP / 2 + t] = i;                       // sorted position (cand's upper half is free)
      kept[32 + (t & 31)] = base;                  // (t < beam <= 32 here; see the launcher)
    }
    n_take += __popcll(bm);
    base += sz4[k];
  }
  lsa_wave_sync();
  for (int t = 0; t < n_take; ++t) {
    const int i = cand[CAP / 2 + t];
    const int b0 = kept[32 + t];
    const int u = spay[i] & 0xffff;
    const int take = min(spay[i] >> 16, K - b0);
    const float uscore = key_float(~(uint32_t)(skey[i] >> 32));
    int o0, o1;
    const int32_t* mem = unit_members(u, o0, o1);
    const int x = o0 + lane;
    const int v = x < o1 ? mem[x] : -1;
    const bool ok = v >= n_sink;
    const int r = __popcll(__ballot(ok) & ((1ull << lane) - 1ull));
    if (ok && r < take) {
      ch_blk[b0 + r] = v;
      ch_sc[b0 + r] = uscore;
    }
  }
  lsa_wave_sync();
  // chosen blocks ascending (the sort space is reused: block in the key, slot as payload)
  int mk = 1;
  while (mk < K) mk <<= 1;
  for (int i = lane; i < mk; i += kWave) {
    skey[i] = i < K ? (uint64_t)(uint32_t)ch_blk[i] : ~(uint64_t)0;
    spay[i] = i;
  }
  lsa_wave_sync();
  if (K > 1) lsa_bitonic_wave(skey, spay, mk);
  lsa_wave_sync();
  // row: sink blocks, chosen blocks, local window, padding
  const int n_s = min(n_sink, c + 1);
  const int l0 = max(n_s, c - n_local + 1);
  const int n_l = max(0, c - l0 + 1);
  const size_t rb = ((size_t)bg * R + row) * NA;
  auto dot_lm = [&](int j) {
    // the landmark row through 16-byte loads, eight at a time, then the products in dimension
    // order
    constexpr int EPV = 16 / sizeof(TIN);
    constexpr int NV = D / EPV, BATCH = NV < 8 ? NV : 8;
    float acc = 0.0f;
#pragma unroll
    for (int t0 = 0; t0 < NV; t0 += BATCH) {
      u32x4 raw[BATCH];
#pragma unroll
      for (int t = 0; t < BATCH; ++t)
        raw[t] = *reinterpret_cast<const u32x4*>(Lg + (size_t)j * D + (t0 + t) * EPV);
#pragma unroll
      for (int t = 0; t < BATCH; ++t) {
        const TIN* x = reinterpret_cast<const TIN*>(&raw[t]);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc = fmaf(qv[(t0 + t) * EPV + e], (float)x[e], acc);
      }
    }
    return acc;
  };
  for (int i = lane; i < NA; i += kWave) {
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

// the widest level, unit list or chosen list of a row (0 if the wave kernel does not apply)
static int lsa_tree_wave_cap(const Shape& s, int seg, int nc, int fan, int beam) {
  if (s.decode || beam > 32) return 0;
  const int ns = s.NB / seg;
  const int need = max(max(s.topk, ns / fan + fan), max(max(beam * fan, beam * nc), beam + seg));
  return need <= 128 ? 128 : need <= kTreeWaveCap ? kTreeWaveCap : 0;
}

bool lsa_tree_shape_ok(const Shape& s, int seg, int nc, int fan, int beam) {
  // the beam search sorts one level's nodes at a time, whatever the number of segments
  if (!lsa_index_ok(seg, nc) || s.topk > kLsaMaxK || fan < 1 || beam < 1 || beam > 64)
    return false;
  const int ns = s.NB / seg;
  return ns / fan + fan <= 1024 && beam * fan <= 1024 && beam * nc <= 1024 &&
         beam + seg <= 1024;
}

hipError_t launch_lsa_tree_centres(const Shape& s, const void* lm, int seg, int fan,
                                   float* seg_c, float* grp_c, hipStream_t st) {
  const int ns = s.NB / seg;
  if (ns == 0) return hipSuccess;
  const int ng = ns / fan;
  dim3 grid(ns, s.B * s.Hkv);
#define BSA_TC(D_, T_)                                                                           \
  hipLaunchKernelGGL((lsa_tree_centres_kernel<D_, T_>), grid, dim3(128), 0, st, (const T_*)lm,    \
                     seg_c, grp_c, s.NB, ns, ng, seg, fan)
  if (s.D == 128) {
    if (s.bf16) BSA_TC(128, bf16);
    else BSA_TC(128, float);
  } else {
    if (s.bf16) BSA_TC(64, bf16);
    else BSA_TC(64, float);
  }
#undef BSA_TC
  return hipGetLastError();
}

hipError_t launch_lsa_tree_select(const Shape& s, const void* q, const void* lm, int seg, int nc,
                                  int fan, int beam, const float* centres, const int32_t* members,
                                  const int32_t* offsets, const float* seg_c, const float* grp_c,
                                  int32_t* idx, float* sc, float* qbar, hipStream_t st) {
  const int ns = s.NB / seg;
  const int cap = lsa_tree_wave_cap(s, seg, nc, fan, beam);
  // the wave kernel forms bf16 rows' selector vectors itself; otherwise the selector pass first
  if (!s.decode && !(cap && s.bf16)) {
    const hipError_t e = launch_selector_vectors(s, q, qbar, st);
    if (e != hipSuccess) return e;
  }
  if (cap) {
    dim3 grid((s.R + 3) / 4, s.B * s.Hkv);
#define BSA_TW(D_, T_, C_, F_)                                                                 \
  hipLaunchKernelGGL((lsa_tree_select_wave_kernel<D_, T_, C_, F_>), grid, dim3(256), 0, st, qbar, \
                     (const T_*)q, (const T_*)lm, centres, members, offsets, seg_c, grp_c, idx,   \
                     sc, s.Hq, s.Hkv, s.G, s.Tq, s.NB, ns, ns / fan, seg, nc, fan, beam, s.R,     \
                     s.topk, s.n_sink, s.n_local, s.NA)
#define BSA_TWC(D_, T_)                                          \
  if (cap == 128) BSA_TW(D_, T_, 128, (sizeof(T_) == 2));        \
  else BSA_TW(D_, T_, kTreeWaveCap, (sizeof(T_) == 2));
    if (s.D == 128) {
      if (s.bf16) {
        BSA_TWC(128, bf16)
      } else {
        BSA_TWC(128, float)
      }
    } else {
      if (s.bf16) {
        BSA_TWC(64, bf16)
      } else {
        BSA_TWC(64, float)
      }
    }
#undef BSA_TWC
#undef BSA_TW
    return hipGetLastError();
  }
  dim3 grid(s.R, s.B * s.Hkv);
#define BSA_TS(D_, T_, K_)                                                                       \
  hipLaunchKernelGGL((lsa_tree_select_kernel<D_, T_, K_>), grid, dim3(256), 0, st, qbar,          \
                     (const T_*)q, (const T_*)lm, centres, members, offsets, seg_c, grp_c, idx, sc, \
                     s.Hq, s.Hkv, s.G, s.NB, ns, ns / fan, seg, nc, fan, beam, s.R,               \
                     s.decode ? s.c_dec : -1, s.topk, s.n_sink, s.n_local, s.NA)
#define BSA_TS_K(D_, T_)                  \
  if (s.topk <= 256) BSA_TS(D_, T_, 256); \
  else BSA_TS(D_, T_, kLsaMaxK);
  if (s.D == 128) {
    if (s.bf16) {
      BSA_TS_K(128, bf16)
    } else {
      BSA_TS_K(128, float)
    }
  } else {
    if (s.bf16) {
      BSA_TS_K(64, bf16)
    } else {
      BSA_TS_K(64, float)
    }
  }
#undef BSA_TS_K
#undef BSA_TS
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// cluster scores of many rows at once (flat index, large indexes)
// ---------------------------------------------------------------------------------------------
// A row of a large flat index scores thousands of centres; one workgroup per row reads every
// centre from L2 once per row.  Here one workgroup scores 64 rows against 64 centres on MFMA, as
// the block scores are formed: each wave takes 32 rows x 32 centres, the selector vectors split
// into three bf16 terms (hi, mid, lo) and the float32 centres likewise, and the six products of
// order 2^-16 or more of the leading one (the three dropped are 2^-24 and below) accumulate in
// float32.  scores[bg][r - row0][u] is written for the
// clusters u of the segments lying wholly at or before row r's last candidate block.
template <int D>
__global__ __launch_bounds__(256) void lsa_unit_scores_kernel(
    const float* __restrict__ qbar, const float* __restrict__ centres, float* __restrict__ scores,
    int R, int NS, int SEG, int NC, int n_local, int row0, int nrows) {
  const int bg = blockIdx.z;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int half = lane / 32, l32 = lane % 32;
  const int UC = NS * NC;
  const int rbase = row0 + (int)blockIdx.x * 64 + (w / 2) * 32;   // this wave's first row
  const int rlast = row0 + nrows - 1;
  if (rbase > rlast) return;                       // no barrier in this kernel
  auto n_units = [&](int r) { return min(NS, max(0, (r - n_local + 1) / SEG)) * NC; };
  const int u0 = (int)blockIdx.y * 64 + (w % 2) * 32;
  if (u0 >= n_units(min(rbase + 31, rlast))) return;   // eligibility only grows with the row
  auto split3 = [](const float* src, bf16x8& h8, bf16x8& m8, bf16x8& l8, bool zero) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = zero ? 0.0f : ((e < 4) ? x0[e] : x1[e - 4]);
      const bf16 h = f2bf(x);
      const float r1 = x - bf2f(h);                // exact in float32
      const bf16 m = f2bf(r1);
      h8[e] = h;
      m8[e] = m;
      l8[e] = f2bf(r1 - bf2f(m));
    }
  };
  const int r = rbase + l32;
  const float* qrow = qbar + ((size_t)bg * R + min(r, rlast)) * D;
  const int u = u0 + l32;
  const float* crow = centres + ((size_t)bg * UC + min(u, UC - 1)) * D;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const int d0 = 16 * st + 8 * half;
    bf16x8 qh, qm, ql, ch, cm, cl;
    split3(qrow + d0, qh, qm, ql, r > rlast);
    split3(crow + d0, ch, cm, cl, u >= UC);
    acc = mfma32(qh, ch, acc);
    acc = mfma32(qm, ch, acc);
    acc = mfma32(ql, ch, acc);
    acc = mfma32(qh, cm, acc);
    acc = mfma32(qm, cm, acc);
    acc = mfma32(qh, cl, acc);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rr = rbase + 8 * (i / 4) + 4 * half + (i % 4);
    if (rr <= rlast && u < n_units(rr))
      scores[((size_t)bg * nrows + (rr - row0)) * UC + u] = acc[i];
  }
}

// candidate blocks of every cluster (members >= n_sink), one thread per cluster: the same for
// every row, so formed once per call for the precomputed-score selection
__global__ __launch_bounds__(256) void lsa_unit_sizes_kernel(const int32_t* __restrict__ members,
                                                             const int32_t* __restrict__ offsets,
                                                             uint16_t* __restrict__ usizes, int NS,
                                                             int SEG, int NC, int n_sink) {
  const int bg = blockIdx.y;
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= NS * NC) return;
  const int sg = u / NC, r = u % NC;
  const size_t sb = (size_t)bg * NS + sg;
  const int o0 = offsets[sb * (NC + 1) + r], o1 = offsets[sb * (NC + 1) + r + 1];
  int size = o1 - o0;
  if (sg * SEG < n_sink) {                         // a segment holding sink blocks
    const int32_t* mem = members + sb * SEG;
    size = 0;
    for (int i = o0; i < o1; ++i) size += mem[i] >= n_sink;
  }
  usizes[(size_t)bg * NS * NC + u] = (uint16_t)size;
}

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------
bool lsa_index_ok(int seg, int nc) { return seg >= 1 && seg <= kLsaMaxSeg && nc >= 1 && nc <= seg; }

// the flat selection sorts every unit of a row at once
bool lsa_shape_ok(const Shape& s, int seg, int nc) {
  if (!lsa_index_ok(seg, nc)) return false;
  const int ns = s.NB / seg;
  if ((int64_t)ns * nc + seg > kLsaMaxUnits) return false;
  return s.topk <= kLsaMaxK;
}

// segments seg0 .. NS-1 (seg0 > 0: the segments completed since the index was last updated)
hipError_t launch_lsa_build(const Shape& s, const void* lm, int seg, int nc, float* centres,
                            int32_t* members, int32_t* offsets, int32_t* merges,
                            hipStream_t st, int seg0) {
  const int ns = s.NB / seg;
  if (ns <= seg0) return hipSuccess;
  dim3 grid(ns - seg0, s.B * s.Hkv);
#define BSA_WARD(D_, T_)                                                                     \
  hipLaunchKernelGGL((lsa_ward_kernel<D_, T_>), grid, dim3(256), 0, st, (const T_*)lm, centres, \
                     members, offsets, merges, s.NB, ns, seg, nc, seg0)
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

// workspace behind the selector vectors: the clusters' candidate counts (at most NB per
// (sequence, kv group)), then a buffer of precomputed cluster scores
static size_t lsa_ws_sizes_bytes(const Shape& s) {
  return ((size_t)s.B * s.Hkv * s.NB * sizeof(uint16_t) + 255) & ~(size_t)255;
}
size_t lsa_ws_score_bytes(const Shape& s) {
  if (s.decode) return 0;
  const size_t full = (size_t)s.B * s.Hkv * s.R * s.NB * sizeof(float);
  return lsa_ws_sizes_bytes(s) + (((full < kLsaScoreBuf ? full : kLsaScoreBuf) + 255) & ~(size_t)255);
}

hipError_t launch_lsa_select(const Shape& s, const void* q, const void* lm, int seg, int nc,
                             const float* centres, const int32_t* members,
                             const int32_t* offsets, int32_t* idx, float* sc, float* qbar,
                             size_t ws_bytes, hipStream_t st) {
  if (!s.decode) {
    const hipError_t e = launch_selector_vectors(s, q, qbar, st);
    if (e != hipSuccess) return e;
  }
  const int ns = s.NB / seg;
  const int uc = ns * nc;                        // cluster units of a row at most
  const int units = uc + seg;
  const bool small_k = s.topk <= 256;
  // large indexes: rows' cluster scores on MFMA first, in chunks of rows that fit the score
  // buffer behind the selector vectors in the workspace
  const size_t qb = s.decode ? 0 : select_ws_qbar_bytes(s);
  const size_t szb = s.decode ? 0 : lsa_ws_sizes_bytes(s);
  const size_t buf = ws_bytes > qb + szb ? ws_bytes - qb - szb : 0;
  const size_t per_row = (size_t)s.B * s.Hkv * uc * sizeof(float);
  const int chunk = (!s.decode && uc > 1024 && per_row > 0)
                        ? (int)std::min<size_t>(buf / per_row, (size_t)s.R) : 0;
  uint16_t* usizes = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(qbar) + qb);
  float* upre = reinterpret_cast<float*>(reinterpret_cast<char*>(qbar) + qb + szb);
  const int nchunks = chunk >= 64 ? (s.R + chunk - 1) / chunk : 1;
  if (chunk >= 64)
    hipLaunchKernelGGL(lsa_unit_sizes_kernel, dim3((uc + 255) / 256, s.B * s.Hkv), dim3(256), 0,
                       st, members, offsets, usizes, ns, seg, nc, s.n_sink);
  for (int ci = 0; ci < nchunks; ++ci) {
    const bool pre = chunk >= 64;
    const int row0 = pre ? ci * chunk : 0;
    const int nrows = pre ? std::min(chunk, s.R - row0) : s.R;
    if (pre) {
      dim3 g1((nrows + 63) / 64, (uc + 63) / 64, s.B * s.Hkv);
      if (s.D == 128)
        hipLaunchKernelGGL(lsa_unit_scores_kernel<128>, g1, dim3(256), 0, st, qbar, centres, upre,
                           s.R, ns, seg, nc, s.n_local, row0, nrows);
      else
        hipLaunchKernelGGL(lsa_unit_scores_kernel<64>, g1, dim3(256), 0, st, qbar, centres, upre,
                           s.R, ns, seg, nc, s.n_local, row0, nrows);
    }
    dim3 grid(nrows, s.B * s.Hkv);
#define BSA_LSEL(D_, T_, U_, K_)                                                                 \
  if (pre)                                                                                       \
    hipLaunchKernelGGL((lsa_select_kernel<D_, T_, U_, K_, true>), grid, dim3(256), 0, st, qbar,   \
                       (const T_*)q, (const T_*)lm, centres, members, offsets, idx, sc, s.Hq,     \
                       s.Hkv, s.G, s.NB, ns, seg, nc, s.R, s.decode ? s.c_dec : -1, s.topk,        \
                       s.n_sink, s.n_local, s.NA, upre, usizes, row0, nrows);                      \
  else                                                                                           \
    hipLaunchKernelGGL((lsa_select_kernel<D_, T_, U_, K_, false>), grid, dim3(256), 0, st, qbar,  \
                       (const T_*)q, (const T_*)lm, centres, members, offsets, idx, sc, s.Hq,     \
                       s.Hkv, s.G, s.NB, ns, seg, nc, s.R, s.decode ? s.c_dec : -1, s.topk,        \
                       s.n_sink, s.n_local, s.NA, nullptr, nullptr, 0, nrows)
#define BSA_LSEL_CAP(D_, T_)                                    \
  if (units <= 1024 && small_k) BSA_LSEL(D_, T_, 1024, 256);    \
  else if (units <= 4608 && small_k) BSA_LSEL(D_, T_, 4608, 256); \
  else if (small_k) BSA_LSEL(D_, T_, kLsaMaxUnits, 256);        \
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
  }
  return hipGetLastError();
}

}  // namespace bsa
