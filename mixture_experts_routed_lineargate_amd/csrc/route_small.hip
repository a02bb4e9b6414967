// Routing of a small batch (at most 32 tokens) in one launch: the router's
// partial logits, the top-k with the RMSNorm factor and the fp16 input planes,
// and the grouping -- the steps of a batched layer before the expert FFN.  As
// three launches (router partials, top-k, grouping) they cost ~24 us at 32
// tokens, mostly launch and drain; here the workgroups hand data over through
// tagged 64-bit words at agent scope, as the decode kernels do
// (decode_common.hpp).  The arithmetic and its order are those of the separate
// kernels: 64-row slices of d_model summed in slice order.
//
//  R  workgroup b: partial logits over slice s = b % NS (64 rows of d_model) of
//     the tokens of group b / NS (8 tokens a group), and the slice's sums of
//     x^2; published.
//  S  workgroup t < T: gathers token t's partials and sums of squares, forms
//     inv = 1/rms (with MOE_F_PRENORM, else 1), logits = inv * sum + bias, the
//     top-k and renormalised weights (lower index wins ties), and the token's
//     input planes inv * x = hi + lo; publishes its k ids.
//  G  workgroup 0: gathers every token's ids and groups them (histogram, scan,
//     stable scatter), then advances the launch counter.
//
// Every word carries the launch's tag (launch counter + 1), so words of earlier
// launches are never taken for this one.  The counter is advanced by workgroup 0
// at its end: by then every workgroup has read it (workgroup 0 has seen every
// token's ids, and token t's workgroup had seen the partials of every slice of
// t's group, so every workgroup had published).  Every wait draws on a per-thread poll budget, so a launch
// always ends; a timeout sets the error word.
#include "decode_common.hpp"
#include "topk_select.hpp"

namespace moe {
namespace rs {

using dec::SPIN_LIMIT;
using dec::gather_fn;
using dec::publish;

constexpr int NT = 512;
constexpr int SL = 64;              // rows of d_model per slice
constexpr int NS_MAX = 32;          // slices (d_model <= 2048)
constexpr int TMAX = 32;            // tokens
constexpr int EMAX = 128;           // experts (two logits per lane of one wavefront)
constexpr int EP = 136;             // words per (slice, token): E partials, sum of squares at E
constexpr int KMAX = 8;
constexpr int TPG = 8;             // tokens per group in R (workgroups: slices x groups)
constexpr int TQ = TPG * EMAX / NT;    // tokens per thread in R
constexpr int QW = (NS_MAX * (EMAX + 1) + NT - 1) / NT;   // gathered words per thread in S
static_assert(TPG * SL % NT == 0 && SL * EMAX % NT == 0 && 2048 / 4 % NT == 0 && TPG <= NT &&
                  EMAX + 1 <= EP && TMAX * KMAX <= NT && TQ * (NT / EMAX) == TPG && NT == 4 * EMAX &&
                  EMAX == 2 * WAVE,
              "shape");

struct Args {
  const float* x;                   // [T][D]
  const float* G;                   // [D][E]
  const float* bias;                // [E] or null
  int T, D, E, k;
  int prenorm;
  int32_t* ids;                     // [T][k]
  float* w;                         // [T][k]
  float* inv;                       // [T] or null
  _Float16* xhi;                    // [T][D]
  _Float16* xlo;                    // [T][D] or null
  int32_t* offsets;                 // [E+1]
  int32_t* rows;                    // [T*k]
  uint64_t* xp;                     // [NS_MAX][TMAX][EP] partial logits and sums of squares
  uint64_t* xi;                     // [TMAX][KMAX] ids
  uint32_t* epoch;                  // launch counter
  uint32_t* err;                    // poll timeout flag
};

__global__ __launch_bounds__(NT) void route_small_kernel(Args p) {
  __shared__ __attribute__((aligned(16))) float xs[TPG][SL + 4];    // rows 16-byte aligned
  __shared__ float gs[SL][EMAX];
  __shared__ float pl[NS_MAX * (EMAX + 1)];
  __shared__ __attribute__((aligned(16))) float lgt[EMAX];
  __shared__ int top[KMAX];
  __shared__ int sids[KMAX];
  __shared__ int cnt[EMAX];
  __shared__ int base[EMAX];
  __shared__ int wcnt[NT / WAVE][EMAX];

  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int b = blockIdx.x, ns = p.D / SL;
  const int s = b % ns, t0 = (b / ns) * TPG;     // R: slice, first token of the group
  const int T = p.T, D = p.D, E = p.E, k = p.k;
  uint32_t budget = SPIN_LIMIT;
  const uint32_t tg = __hip_atomic_load(p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  // the bias is read now: read at the top-k it would cost a memory latency there
  float bv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) bv[i] = p.bias ? p.bias[min(i * WAVE + lane, E - 1)] : 0.f;

  // ---- R: partial logits of slice s ----
  // (loads first, all unconditional: clamped rows and columns, masked at use)
  constexpr int XL = TPG * SL / NT;
  float xv[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int i = j * NT + tid, t = min(t0 + i / SL, T - 1), c = i % SL;
    xv[j] = p.x[(int64_t)t * D + s * SL + c];
  }
  constexpr int GL = SL * EMAX / NT;
  float gv[GL];
#pragma unroll
  for (int j = 0; j < GL; ++j) {
    const int i = j * NT + tid, c = i / EMAX, ee = i % EMAX;
    gv[j] = p.G[(int64_t)(s * SL + c) * E + min(ee, E - 1)];
  }
  // token b's input row, needed in S only after the partials arrive
  constexpr int XR = 2048 / 4 / NT;
  float4 xr[XR];
  {
    const int tt = min(b, T - 1);
#pragma unroll
    for (int j = 0; j < XR; ++j)
      xr[j] = *(const float4*)(p.x + (int64_t)tt * D + 4 * min(j * NT + tid, D / 4 - 1));
  }
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int i = j * NT + tid;
    xs[i / SL][i % SL] = t0 + i / SL < T ? xv[j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < GL; ++j) {
    const int i = j * NT + tid;
    gs[i / EMAX][i % EMAX] = gv[j];
  }
  __syncthreads();
  const int e = tid % EMAX, th = tid / EMAX;     // expert, token group (tokens TQ th ..)
  float acc[TQ];
#pragma unroll
  for (int i = 0; i < TQ; ++i) acc[i] = 0.f;
#pragma unroll 2
  for (int c = 0; c < SL; c += 4) {
    const float g[4] = {gs[c][e], gs[c + 1][e], gs[c + 2][e], gs[c + 3][e]};
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      const float4 xq = *(const float4*)&xs[th * TQ + i][c];
      acc[i] = fmaf(xq.x, g[0], acc[i]);
      acc[i] = fmaf(xq.y, g[1], acc[i]);
      acc[i] = fmaf(xq.z, g[2], acc[i]);
      acc[i] = fmaf(xq.w, g[3], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < TQ; ++i) {
    const int t = t0 + th * TQ + i;
    if (t < T && e < E) publish(p.xp + ((int64_t)s * TMAX + t) * EP + e, tg, acc[i]);
  }
  if (tid < TPG && t0 + tid < T) {
    float sq = 0.f;
#pragma unroll
    for (int c = 0; c < SL; ++c) sq = fmaf(xs[tid][c], xs[tid][c], sq);
    publish(p.xp + ((int64_t)s * TMAX + t0 + tid) * EP + E, tg, sq);
  }

  // ---- S: token b ----
  if (b < T) {
    const int nw = ns * (E + 1);
    float vals[QW];
    gather_fn<QW>(
        [=](int i) {
          const int q = min(i * NT + tid, nw - 1);
          return p.xp + ((int64_t)(q / (E + 1)) * TMAX + b) * EP + q % (E + 1);
        },
        tg, p.err, budget, vals);
#pragma unroll
    for (int i = 0; i < QW; ++i)
      if (i * NT + tid < nw) pl[i * NT + tid] = vals[i];
    __syncthreads();
    // logits: thread e < E sums its expert's partials in slice order, and (every
    // one of them, the same sums in the same order) the sums of squares for inv;
    // the slots past E hold NaN, which no comparison counts
    float ssq = 0.f;
#pragma unroll 8
    for (int q = 0; q < ns; ++q) ssq += pl[q * (E + 1) + E];
    const float inv = p.prenorm ? 1.0f / sqrtf(ssq / (float)D + PRENORM_EPS) : 1.0f;
    if (tid < EMAX) {
      float l = __builtin_nanf("");
      if (tid < E) {
        float a = 0.f;
#pragma unroll 8
        for (int q = 0; q < ns; ++q) a += pl[q * (E + 1) + tid];   // slice order
        l = p.bias ? fmaf(a, inv, bv[wave]) : a * inv;   // bias of expert wave * WAVE + lane
      }
      lgt[tid] = l;
    }
    if (tid < KMAX) top[tid] = -1;
    if (p.inv && tid == 0) p.inv[b] = inv;
    __syncthreads();
    // the top-k by rank counting over the workgroup, four threads a logit: another
    // logit outranks e if it is larger, or equal with a lower index, so expert e is
    // selected iff fewer than k logits outrank it.  A first pass counts only the
    // logits >= lgt[e] (one compare a pair); less one (e itself) that is e's rank
    // whenever no other logit equals it.  m >= 2 equal logits under c larger ones
    // all claim slot c + m - 1 and leave slot c empty, so when the k slots are all
    // filled no tie reaches the top k and the slots hold the exact ranks.
    // Otherwise a second pass ranks with the full comparison, every slot preset to
    // its own index, so the ids are in [0, E) whatever the logits hold.
    {
      const int e = tid >> 2, q = tid & 3;
      const float le = lgt[e];
      float4 v[EMAX / 16];
#pragma unroll
      for (int i = 0; i < EMAX / 16; ++i) v[i] = *(const float4*)(lgt + (EMAX / 4) * q + 4 * i);
      int ge = 0;
#pragma unroll
      for (int i = 0; i < EMAX / 16; ++i)
        ge += (v[i].x >= le) + (v[i].y >= le) + (v[i].z >= le) + (v[i].w >= le);
      ge += dpp<DPP_QUAD_1032>(ge);
      ge += dpp<DPP_QUAD_2301>(ge);
      if (q == 0 && e < E && ge >= 1 && ge <= k) top[ge - 1] = e;
    }
    __syncthreads();
    int hole = 0;
    for (int r = 0; r < k; ++r) hole |= top[r] < 0;
    if (hole) {                                       // uniform: every thread read the same slots
      __syncthreads();
      if (tid < KMAX) top[tid] = tid;
      __syncthreads();
      const int e = tid >> 2, q = tid & 3;
      int cnt = 0;
      if (e < E) {
        const float le = lgt[e];
#pragma unroll 8
        for (int i = 0; i < EMAX / 4; ++i) {
          const int j = (EMAX / 4) * q + i;
          const float lj = lgt[j];
          cnt += (j < E) & ((lj > le) | ((lj == le) & (j < e)));
        }
      }
      cnt += dpp<DPP_QUAD_1032>(cnt);
      cnt += dpp<DPP_QUAD_2301>(cnt);
      if (q == 0 && e < E && cnt < k) top[cnt] = e;
      __syncthreads();
    }
    if (wave == 0) {
      // renormalised softmax over the winners: lane r < k takes winner r (rank
      // order); the denominator is summed in rank order; outputs in ascending id
      const int me = min(max(top[min(lane, k - 1)], 0), E - 1);
      const float lmax = lgt[min(max(top[0], 0), E - 1)];
      const float ex = expf(lgt[me] - lmax);
      float den = 0.f;
      for (int r = 0; r < k; ++r) den += __shfl(ex, r, WAVE);
      int rank = 0;
      for (int r = 0; r < k; ++r) rank += top[r] < me;
      rank = min(rank, k - 1);
      if (lane < k) {
        p.ids[b * k + rank] = me;
        sids[rank] = me;
        p.w[b * k + rank] = ex / den;
      }
    }
    // input planes of token b, in the planes' order (element by element: a packed
    // conversion would round ties unlike the other kernels that write planes)
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int d = 4 * (j * NT + tid);
      if (d >= D) break;
      const float u[4] = {xr[j].x * inv, xr[j].y * inv, xr[j].z * inv, xr[j].w * inv};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 hi = (_Float16)u[i];
        p.xhi[(int64_t)b * D + plane_pos(d + i)] = hi;
        if (p.xlo) p.xlo[(int64_t)b * D + plane_pos(d + i)] = (_Float16)(u[i] - (float)hi);
      }
    }
    __syncthreads();                                  // sids written by wavefront 0
    if (tid < k) publish(p.xi + b * KMAX + tid, tg, __int_as_float(sids[tid]));
  }

  // ---- G: grouping of the T*k ids (workgroup 0) ----
  if (b == 0) {
    const int N = T * k;
    float idv[1];
    gather_fn<1>([=](int) { const int i = min(tid, N - 1); return p.xi + (i / k) * KMAX + i % k; },
                 tg, p.err, budget, idv);
    const bool valid = tid < N;
    const int ev = valid ? min(max(__float_as_int(idv[0]), 0), E - 1) : -1;
    for (int x = tid; x < EMAX; x += NT) cnt[x] = 0;
    for (int x = tid; x < (NT / WAVE) * EMAX; x += NT) (&wcnt[0][0])[x] = 0;
    __syncthreads();
    // rank among the equal ids of this wavefront (ballot multisplit), per-wave counts
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((ev >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
    const int rank = __popcll(m & below);
    if (valid && rank == 0) {
      wcnt[wave][ev] = __popcll(m);
      atomicAdd(&cnt[ev], __popcll(m));
    }
    __syncthreads();
    if (wave == 0) {                                  // offsets: exclusive scan of the counts
      const int a = 2 * lane < E ? cnt[2 * lane] : 0;
      const int b = 2 * lane + 1 < E ? cnt[2 * lane + 1] : 0;
      int incl = a + b;
#pragma unroll
      for (int off = 1; off < WAVE; off <<= 1) {
        const int o = __shfl_up(incl, off, WAVE);
        if (lane >= off) incl += o;
      }
      const int excl = incl - a - b;
      if (2 * lane < E) {
        base[2 * lane] = excl;
        p.offsets[2 * lane] = excl;
      }
      if (2 * lane + 1 < E) {
        base[2 * lane + 1] = excl + a;
        p.offsets[2 * lane + 1] = excl + a;
      }
      if (lane == WAVE - 1) p.offsets[E] = incl;
    }
    __syncthreads();
    if (valid) {
      int pos = base[ev] + rank;
      for (int w2 = 0; w2 < wave; ++w2) pos += wcnt[w2][ev];
      p.rows[pos] = tid;
    }
    if (tid == 0) __hip_atomic_store(p.epoch, tg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace rs

bool route_small_supported(int64_t T, int D, int E, int k) {
  return T >= 1 && T <= rs::TMAX && E <= rs::EMAX && k <= rs::KMAX && D % rs::SL == 0 &&
         D / rs::SL <= rs::NS_MAX && T <= D / rs::SL;
}

hipError_t launch_route_small(const float* x, int64_t T, int D, const float* G, const float* bias,
                              int E, int k, bool prenorm, int32_t* ids, float* w, float* inv,
                              _Float16* xhi, _Float16* xlo, int32_t* offsets, int32_t* rows,
                              const Workspace& ws, hipStream_t s) {
  rs::Args a{};
  a.x = x;
  a.G = G;
  a.bias = bias;
  a.T = (int)T;
  a.D = D;
  a.E = E;
  a.k = k;
  a.prenorm = prenorm ? 1 : 0;
  a.ids = ids;
  a.w = w;
  a.inv = inv;
  a.xhi = xhi;
  a.xlo = xlo;
  a.offsets = offsets;
  a.rows = rows;
  // exchange words in the workspace's sync region, clear of the decode kernels' regions
  char* sync = (char*)ws.sync;
  a.err = ws.sync + ERR_WORD_OFF / sizeof(uint32_t);
  a.epoch = (uint32_t*)(sync + 8192);
  a.xp = (uint64_t*)(sync + ROUTE_SYNC_OFF);
  a.xi = (uint64_t*)(sync + ROUTE_SYNC_OFF + (size_t)rs::NS_MAX * rs::TMAX * rs::EP * 8);
  static_assert(ROUTE_SYNC_OFF + (size_t)rs::NS_MAX * rs::TMAX * rs::EP * 8 +
                        (size_t)rs::TMAX * rs::KMAX * 8 <= SYNC_BYTES,
                "sync region");
  const int groups = (int)((T + rs::TPG - 1) / rs::TPG);
  hipLaunchKernelGGL(rs::route_small_kernel, dim3((unsigned)(D / rs::SL * groups)), dim3(rs::NT), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace moe
