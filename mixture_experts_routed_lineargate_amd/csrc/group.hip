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

// Single pass for GT < N <= FC * GT entries and up to FE experts (the prefill
// microbatches).  The ids stay in registers (thread t holds
// entries c * GT + t); the per-(chunk, wavefront) counts of each expert come
// from the same wave multisplit; one pass then turns them into exclusive
// prefixes in (chunk, wavefront) order, expert by expert (thread 8e + c owns
// expert e, chunk c: a serial prefix over the 16 wavefronts, then a scan over
// the 8 chunk threads), and the expert totals are scanned into the offsets.
// The position of entry i is offsets[e] + prefix(e, chunk, wavefront) + rank,
// the same stable order as above.
constexpr int FC = 8;             // chunks of GT entries
constexpr int FE = 128;           // experts
constexpr int FS = FC * GW + 1;   // LDS stride per expert (odd: spreads the banks)
static_assert(FC * FE == GT, "one thread per (expert, chunk)");

__global__ __launch_bounds__(GT) void group_fast_kernel(const int32_t* __restrict__ ids, int N,
                                                        int E, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ rows) {
  __shared__ int cnt[FE * FS];    // [e][c * GW + w]: count, then exclusive prefix
  __shared__ int tot[FE];
  __shared__ int base[FE + 1];
  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  int ev[FC];
#pragma unroll
  for (int c = 0; c < FC; ++c) {
    const int i = c * GT + tid;
    ev[c] = i < N ? ids[i] : -1;
  }
  for (int j = tid; j < FE * FS; j += GT) cnt[j] = 0;
  __syncthreads();

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
  int rank[FC];
#pragma unroll
  for (int c = 0; c < FC; ++c) {
    const int e = ev[c];
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    rank[c] = __popcll(m & below);
    if (valid && rank[c] == 0) cnt[e * FS + c * GW + wave] = __popcll(m);
  }
  __syncthreads();

  {
    const int e = tid / FC, c = tid % FC;
    int* row = cnt + e * FS + c * GW;
    int v[GW];
#pragma unroll
    for (int w = 0; w < GW; ++w) v[w] = row[w];
    int run = 0;
#pragma unroll
    for (int w = 0; w < GW; ++w) {
      const int x = v[w];
      v[w] = run;
      run += x;
    }
    int incl = run;                                   // scan over the FC chunk threads of e
#pragma unroll
    for (int off = 1; off < FC; off <<= 1) {
      const int o = __shfl_up(incl, off, FC);
      if (c >= off) incl += o;
    }
    const int excl = incl - run;
#pragma unroll
    for (int w = 0; w < GW; ++w) row[w] = v[w] + excl;
    if (c == FC - 1) tot[e] = incl;
  }
  __syncthreads();

  if (wave == 0) {                                    // offsets: exclusive scan of the totals
    const int a = 2 * lane < E ? tot[2 * lane] : 0;
    const int b = 2 * lane + 1 < E ? tot[2 * lane + 1] : 0;
    int incl = a + b;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
      const int o = __shfl_up(incl, off, WAVE);
      if (lane >= off) incl += o;
    }
    const int excl = incl - a - b;
    if (2 * lane < E) {
      base[2 * lane] = excl;
      offsets[2 * lane] = excl;
    }
    if (2 * lane + 1 < E) {
      base[2 * lane + 1] = excl + a;
      offsets[2 * lane + 1] = excl + a;
    }
    if (lane == WAVE - 1) offsets[E] = incl;
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < FC; ++c) {
    const int e = ev[c];
    if ((unsigned)e < (unsigned)E)
      rows[base[e] + cnt[e * FS + c * GW + wave] + rank[c]] = c * GT + tid;
  }
}

hipError_t launch_group(const int32_t* ids, int64_t N, int E, int32_t* offsets, int32_t* rows,
                        hipStream_t s) {
  // one chunk or less: the chunked kernel has the lower fixed cost (its LDS
  // footprint is E + GW * E words against FE * FS here)
  if (E <= FE && N > GT && N <= (int64_t)FC * GT) {
    hipLaunchKernelGGL(group_fast_kernel, dim3(1), dim3(GT), 0, s, ids, (int)N, E, offsets, rows);
    return hipGetLastError();
  }
  const size_t lds = (size_t)(E + GW * E) * sizeof(int);
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(GT), lds, s, ids, N, E, offsets, rows);
  return hipGetLastError();
}

}  // namespace moe
