// Compact per-expert grouping: histogram, exclusive scan, stable scatter of
// the flat (token, slot) index.  (Reuse-ordering page, "What changed from the
// first experiment": the existing compact expert grouping is reused without a
// new routing sort.)
//
// One workgroup of 1024 threads.  Stability without atomics in the scatter:
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

hipError_t launch_group(const int32_t* ids, int64_t N, int E, int32_t* offsets, int32_t* rows,
                        hipStream_t s) {
  const size_t lds = (size_t)(E + GW * E) * sizeof(int);
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(GT), lds, s, ids, N, E, offsets, rows);
  return hipGetLastError();
}

}  // namespace moe
