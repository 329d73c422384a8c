// Landmark pooling and selector vectors: coalesced HBM streaming with float64 accumulation.
//
// Landmarks (LSA page, "The index stops scanning the whole context", paragraph 3: neighbouring
// keys are pooled before indexing): lm[b,g,j,:] = mean of k[b,g,t,:] over the tokens of block j,
// rounded once to the input dtype.  Selector vectors: qbar[b,g,c,:] = sum over the query heads
// of group g of the mean of q over the tokens of query block c (a decode step is the case of
// one query token), kept in float32.
//
// Accumulating in float64 makes the bf16 block mean exact before the single rounding: 64
// (or G*64) bf16 values carry 8 significant bits each, so their sum needs far fewer than 53.
#include <algorithm>

#include "bsa_common.hpp"
#include "bsa_internal.hpp"

namespace bsa {

// One workgroup of 256 threads reduces `nrows` rows of D elements.  Row r lives at
// src + row_base(r) * D with row_base(r) = (r / rows_per_head) * head_stride + r % rows_per_head.
// Thread layout: NC column chunks of 16 bytes, 256 / NC row groups.
// Output blocks blk0 + blockIdx.x (blk0 > 0: only the tail of the blocks is recomputed).
template <typename T, typename OUT, int D>
__global__ __launch_bounds__(256) void pool_rows_kernel(const T* __restrict__ src,
                                                        OUT* __restrict__ dst, int T_len,
                                                        int heads_src, int heads_per_group,
                                                        int n_groups, int n_out_blocks, int blk0) {
  constexpr int EPC = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int NC = D / EPC;                // chunks per row
  constexpr int RG = 256 / NC;               // row groups
  __shared__ double red[RG][D];

  const int blk = blk0 + blockIdx.x;         // output block (query block or key block)
  const int grp = blockIdx.y;                // group index within the batch entry
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int chunk = tid % NC;
  const int rg = tid / NC;

  const int t0 = blk * kBlock;
  const int ntok = min(kBlock, T_len - t0);
  const int nrows = ntok * heads_per_group;

  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;

  for (int r = rg; r < nrows; r += RG) {
    const int hh = r / ntok;
    const int t = t0 + r % ntok;
    const int head = grp * heads_per_group + hh;
    const T* row = src + ((size_t)(b * heads_src + head) * T_len + t) * D;
    u32x4 raw = *reinterpret_cast<const u32x4*>(row + chunk * EPC);
    const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += (double)(float)vals[e];
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[rg][chunk * EPC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
    for (int i = 0; i < RG; ++i) s += red[i][tid];
    const double mean = s / (double)ntok;
    OUT* o = dst + ((size_t)(b * n_groups + grp) * n_out_blocks + blk) * D + tid;
    if constexpr (sizeof(OUT) == 2) {
      *o = f64_to_bf16_rne(mean);
    } else {
      *o = (float)mean;  // round-to-nearest-even float64 -> float32
    }
  }
}

// Landmarks of a paged cache: block j of sequence b (page table[b * NB + j] of the pool
// [n_pages, Hkv, 64, D]) averages its first min(64, len_b - 64 j) tokens, len_b = lens[b]
// clamped to 1 .. NB * 64; blocks past the end of a sequence are written as zeros.  Same float64
// accumulation and single rounding as above.
// n_new > 0 (refresh after appending n_new tokens to every sequence): workgroup x of sequence b
// recomputes block (len_b - n_new) / 64 + x, the blocks holding the last n_new tokens, and skips
// blocks past the sequence's last one; nothing else is written.  n_new == 0: every block.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_paged_kernel(const T* __restrict__ pool,
                                                         T* __restrict__ dst,
                                                         const int32_t* __restrict__ table,
                                                         const int32_t* __restrict__ lens, int Hkv,
                                                         int NB, int n_pages, int n_new) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int NC = D / EPC;
  constexpr int RG = 256 / NC;
  __shared__ double red[RG][D];
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int chunk = tid % NC, rg = tid / NC;
  const int len = min(max(lens[b], 1), NB * kBlock);
  int j = blockIdx.x;
  if (n_new > 0) {
    j += max(len - n_new, 0) / kBlock;
    if (j > (len - 1) / kBlock) return;                // past this sequence's last block
  }
  const int ntok = min(kBlock, len - j * kBlock);      // <= 0: block past the end
  T* o = dst + ((size_t)(b * Hkv + g) * NB + j) * D;
  if (ntok <= 0) {
    for (int d = tid; d < D; d += 256) o[d] = (T)0.0f;
    return;
  }
  const int pg = min(max(table[(size_t)b * NB + j], 0), n_pages - 1);
  const T* blk = pool + ((size_t)pg * Hkv + g) * kBlock * D;
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
  for (int r = rg; r < ntok; r += RG) {
    u32x4 raw = *reinterpret_cast<const u32x4*>(blk + (size_t)r * D + chunk * EPC);
    const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += (double)(float)vals[e];
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[rg][chunk * EPC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double sum = 0.0;
    for (int i = 0; i < RG; ++i) sum += red[i][tid];
    const double mean = sum / (double)ntok;
    if constexpr (sizeof(T) == 2) o[tid] = f64_to_bf16_rne(mean);
    else o[tid] = (float)mean;
  }
}

hipError_t launch_pool_landmarks_paged(const Shape& s, const void* k_pool, const Pages& pg,
                                       void* lm, hipStream_t st, int n_new) {
  // a refresh of the last n_new tokens touches at most ceil(n_new / 64) + 1 blocks
  const int nx = n_new > 0 ? std::min(s.NB, (n_new + kBlock - 1) / kBlock + 1) : s.NB;
  dim3 grid(nx, s.Hkv, s.B);
#define BSA_PPOOL(T_, D_)                                                                   \
  hipLaunchKernelGGL((pool_paged_kernel<T_, D_>), grid, dim3(256), 0, st, (const T_*)k_pool, \
                     (T_*)lm, pg.table, pg.lens, s.Hkv, s.NB, pg.n_pages, n_new)
  if (s.bf16) {
    if (s.D == 128) BSA_PPOOL(bf16, 128);
    else BSA_PPOOL(bf16, 64);
  } else {
    if (s.D == 128) BSA_PPOOL(float, 128);
    else BSA_PPOOL(float, 64);
  }
#undef BSA_PPOOL
  return hipGetLastError();
}

template <typename T, typename OUT>
static hipError_t launch_pool_t(const void* src, void* dst, int B, int heads_src, int groups,
                                int heads_per_group, int T_len, int D, hipStream_t st,
                                int blk0 = 0) {
  const int nb = (T_len + kBlock - 1) / kBlock;
  dim3 grid(nb - blk0, groups, B);
  if (D == 128) {
    hipLaunchKernelGGL((pool_rows_kernel<T, OUT, 128>), grid, dim3(256), 0, st,
                       (const T*)src, (OUT*)dst, T_len, heads_src, heads_per_group, groups, nb,
                       blk0);
  } else {
    hipLaunchKernelGGL((pool_rows_kernel<T, OUT, 64>), grid, dim3(256), 0, st,
                       (const T*)src, (OUT*)dst, T_len, heads_src, heads_per_group, groups, nb,
                       blk0);
  }
  return hipGetLastError();
}

// n_new > 0: only the blocks holding the last n_new of the Tk tokens
hipError_t launch_pool_landmarks(const Shape& s, const void* k, void* lm, hipStream_t st,
                                 int n_new) {
  const int blk0 = n_new > 0 ? std::max(s.Tk - n_new, 0) / kBlock : 0;
  if (s.bf16)
    return launch_pool_t<bf16, bf16>(k, lm, s.B, s.Hkv, s.Hkv, 1, s.Tk, s.D, st, blk0);
  return launch_pool_t<float, float>(k, lm, s.B, s.Hkv, s.Hkv, 1, s.Tk, s.D, st, blk0);
}

hipError_t launch_selector_vectors(const Shape& s, const void* q, float* qbar, hipStream_t st) {
  if (s.bf16)
    return launch_pool_t<bf16, float>(q, qbar, s.B, s.Hq, s.Hkv, s.G, s.Tq, s.D, st);
  return launch_pool_t<float, float>(q, qbar, s.B, s.Hq, s.Hkv, s.G, s.Tq, s.D, st);
}

}  // namespace bsa
