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

bool lsa_tree_shape_ok(const Shape& s, int seg, int nc, int fan, int beam) {
  if (!lsa_shape_ok(s, seg, nc) || fan < 1 || beam < 1 || beam > 64) return false;
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
  if (!s.decode) {
    const hipError_t e = launch_selector_vectors(s, q, qbar, st);
    if (e != hipSuccess) return e;
  }
  const int ns = s.NB / seg;
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
