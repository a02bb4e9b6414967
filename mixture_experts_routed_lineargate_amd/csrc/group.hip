// Compact per-expert grouping: histogram, exclusive scan, stable scatter of
// the flat (token, slot) index.  (Reuse-ordering page, "What changed from the
// first experiment": the existing compact expert grouping is reused without a
// new routing sort.)
//
// Up to 1024 entries (or beyond the chunk-parallel kernel's limits): one
// workgroup of 1024 threads.  Stability without atomics in the scatter:
// inside a wavefront, lanes holding the same expert are found with one ballot
// per expert-id bit (a wave multisplit), a lane's rank is the popcount of the
// equal lanes below it; wave totals are scanned across the 16 wavefronts per
// expert in wave order, and a running per-expert cursor carries across
// 1024-entry chunks.  Every position therefore equals offsets[e] + (number of
// earlier flat indices with expert e), independent of scheduling.
#include "internal.hpp"

namespace moe {

constexpr int GT = 1024;          // threads
constexpr int GW = GT / WAVE;     // wavefronts

__global__ __launch_bounds__(GT) void group_kernel(const int32_t* __restrict__ ids, int64_t N,
                                                   int E, int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ rows) {
  extern __shared__ int smem[];
  int* cursor = smem;            // [E]
  int* wcnt = smem + E;          // [GW][E]
  __shared__ int scan_tmp[GW];
  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  for (int e = tid; e < E; e += GT) cursor[e] = 0;
  __syncthreads();
  for (int64_t i = tid; i < N; i += GT) {
    const int e = ids[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cursor[e], 1);
  }
  __syncthreads();

  // Exclusive scan of the counts (E <= 1024: one value per thread).
  {
    const int c = tid < E ? cursor[tid] : 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
      const int o = __shfl_up(incl, off, WAVE);
      if (lane >= off) incl += o;
    }
    if (lane == WAVE - 1) scan_tmp[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += scan_tmp[w];
    const int excl = wbase + incl - c;
    __syncthreads();
    if (tid < E) {
      cursor[tid] = excl;
      offsets[tid] = excl;
    }
    if (tid == E - 1) offsets[E] = excl + c;
  }
  __syncthreads();

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
  for (int64_t c0 = 0; c0 < N; c0 += GT) {
    const int64_t i = c0 + tid;
    int e = (i < N) ? ids[i] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    if (!valid) m = 0;
    const int rank = __popcll(m & below);
    for (int j = tid; j < GW * E; j += GT) wcnt[j] = 0;
    __syncthreads();
    if (valid && rank == 0) wcnt[wave * E + e] = __popcll(m);
    __syncthreads();
    for (int x = tid; x < E; x += GT) {
      int run = cursor[x];
      for (int w = 0; w < GW; ++w) {
        const int cnt = wcnt[w * E + x];
        wcnt[w * E + x] = run;
        run += cnt;
      }
      cursor[x] = run;
    }
    __syncthreads();
    if (valid) rows[wcnt[wave * E + e] + rank] = (int32_t)i;
    __syncthreads();
  }
}

// More than one chunk (GT < N <= CMAX * GT entries, up to ME experts): one
// workgroup per 1024-entry chunk and no exchange between them.  Every
// workgroup counts all N entries per (chunk, expert) in LDS; plain counts
// suffice, since the chunk index carries the order.  From them it has the
// expert totals (hence the offsets) and, for each expert, the entries in the
// chunks before its own.  Its own chunk then gets the wave multisplit's stable
// ranks and a prefix over its wavefronts, so entry i lands at
// offsets[e] + (entries of e in earlier chunks) + (in earlier wavefronts of its
// chunk) + (in lower lanes of its wavefront): the same stable order as above.
constexpr int CMAX = 32;          // chunks
constexpr int ME = 256;           // experts
static_assert(ME <= GT && ME == 4 * WAVE, "one thread per expert; the offset scan takes four per lane");

__global__ __launch_bounds__(GT) void group_multi_kernel(const int32_t* __restrict__ ids, int N,
                                                         int E, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ rows) {
  extern __shared__ int smem[];
  const int nch = (N + GT - 1) / GT;
  int* cnt = smem;                // [nch][E] entries per (chunk, expert)
  int* wcnt = cnt + nch * E;      // [GW][E] own chunk: per wavefront, then its prefix
  int* tot = wcnt + GW * E;       // [E]
  int* base = tot + E;            // [E] offsets
  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int b = blockIdx.x;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  for (int j = tid; j < (nch + GW) * E; j += GT) cnt[j] = 0;
  const int i_own = b * GT + tid;
  const int e_own = i_own < N ? ids[i_own] : -1;
  __syncthreads();
  for (int c0 = 0; c0 < nch; c0 += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = (c0 + u) * GT + tid;
      v[u] = i < N ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if ((unsigned)v[u] < (unsigned)E) atomicAdd(&cnt[(c0 + u) * E + v[u]], 1);
  }

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
  const bool valid = (unsigned)e_own < (unsigned)E;
  uint64_t m = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool on = valid && ((e_own >> bit) & 1);
    const uint64_t bb = __ballot(on);
    m &= on ? bb : ~bb;
  }
  const int rank = __popcll(m & below);
  if (valid && rank == 0) wcnt[wave * E + e_own] = __popcll(m);
  __syncthreads();

  if (tid < E) {
    const int e = tid;
    int all = 0, before = 0;
    for (int c = 0; c < nch; ++c) {
      const int x = cnt[c * E + e];
      before += c < b ? x : 0;
      all += x;
    }
    int run = before;
#pragma unroll
    for (int w = 0; w < GW; ++w) {
      const int x = wcnt[w * E + e];
      wcnt[w * E + e] = run;
      run += x;
    }
    tot[e] = all;
  }
  __syncthreads();

  if (wave == 0) {                                    // offsets: exclusive scan of the totals
    int t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = 4 * lane + u < E ? tot[4 * lane + u] : 0;
    const int sum = t[0] + t[1] + t[2] + t[3];
    int incl = sum;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
      const int o = __shfl_up(incl, off, WAVE);
      if (lane >= off) incl += o;
    }
    int run = incl - sum;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * lane + u;
      if (e < E) {
        base[e] = run;
        if (b == 0) offsets[e] = run;
      }
      run += t[u];
    }
    if (b == 0 && lane == WAVE - 1) offsets[E] = incl;
  }
  __syncthreads();
  if (valid) rows[base[e_own] + wcnt[wave * E + e_own] + rank] = i_own;
}

hipError_t launch_group(const int32_t* ids, int64_t N, int E, int32_t* offsets, int32_t* rows,
                        hipStream_t s) {
  if (E <= ME && N > GT && N <= (int64_t)CMAX * GT) {
    const int nch = (int)((N + GT - 1) / GT);
    const size_t lds = (size_t)((nch + GW) * E + 2 * E) * sizeof(int);
    hipLaunchKernelGGL(group_multi_kernel, dim3(nch), dim3(GT), lds, s, ids, (int)N, E, offsets, rows);
    return hipGetLastError();
  }
  const size_t lds = (size_t)(E + GW * E) * sizeof(int);
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(GT), lds, s, ids, N, E, offsets, rows);
  return hipGetLastError();
}

}  // namespace moe
