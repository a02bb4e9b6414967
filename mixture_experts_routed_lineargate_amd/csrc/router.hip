// LinearGate router: logits = x G + b, top-k with lower-index tie-break,
// renormalised softmax weights.  (Evidence page, "Layer-qualified experts":
// learned LinearGate selection; Model card: top-8 of 128 experts.)
#include <float.h>

#include "topk_select.hpp"

namespace moe {

// Number of D-slices the router GEMV/GEMM is split into, so that small T still
// spreads the 1 MiB gate over many CUs.  Each slice is a multiple of 32 rows.
int router_ksplit(int64_t T, int D) {
  const int64_t tiles = T >= 32 ? (T + 31) / 32 : (T + 7) / 8;
  int64_t ks = 512 / (tiles > 0 ? tiles : 1);     // ~two workgroups per CU
  if (ks > 32) ks = 32;            // the top-k pass sums ks partials per logit
  if (ks < 1) ks = 1;
  if (ks > D / 32) ks = D / 32;
  int dchunk = (int)(((D + ks - 1) / ks + 31) / 32 * 32);
  return (D + dchunk - 1) / dchunk;
}

static int router_dchunk(int D, int ks) { return (int)(((D + ks - 1) / ks + 31) / 32 * 32); }

// part[s][t][e] = sum over the s-th D-slice of x[t][d] * G[d][e].
// Block: 256 threads = 128 experts x 2 token halves; TT tokens per block.
template <int TT>
__global__ __launch_bounds__(256) void router_partial_kernel(const float* __restrict__ x, int64_t T,
                                                             int D, const float* __restrict__ G,
                                                             int E, int dchunk,
                                                             float* __restrict__ part,
                                                             float* __restrict__ ssq) {
  constexpr int DC = 32;
  constexpr int TH = TT / 2;
  __shared__ float xs[TT][DC];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int s = blockIdx.y;
  const int d0 = s * dchunk;
  const int d1 = min(D, d0 + dchunk);
  const int el = tid & 127, half = tid >> 7;
  float sq[TH];                                   // sum of x^2 over the slice
#pragma unroll
  for (int i = 0; i < TH; ++i) sq[i] = 0.f;
  for (int ec = 0; ec < E; ec += 128) {
    const int e = ec + el;
    float acc[TH];
#pragma unroll
    for (int i = 0; i < TH; ++i) acc[i] = 0.f;
    for (int dd = d0; dd < d1; dd += DC) {
      __syncthreads();
      for (int i = tid; i < TT * DC; i += 256) {
        const int tt = i / DC, c = i % DC;
        const int64_t t = t0 + tt;
        xs[tt][c] = (t < T) ? x[t * D + dd + c] : 0.f;
      }
      __syncthreads();
      if (ec == 0) {
        for (int c = 0; c < DC; ++c)
#pragma unroll
          for (int i = 0; i < TH; ++i) sq[i] = fmaf(xs[half * TH + i][c], xs[half * TH + i][c], sq[i]);
      }
      if (e < E) {
#pragma unroll 8
        for (int c = 0; c < DC; ++c) {
          const float g = G[(int64_t)(dd + c) * E + e];
#pragma unroll
          for (int i = 0; i < TH; ++i) acc[i] = fmaf(xs[half * TH + i][c], g, acc[i]);
        }
      }
    }
    if (e < E) {
#pragma unroll
      for (int i = 0; i < TH; ++i) {
        const int64_t t = t0 + half * TH + i;
        if (t < T) part[((int64_t)s * T + t) * E + e] = acc[i];
      }
    }
  }
  if (ssq && el == 0) {
#pragma unroll
    for (int i = 0; i < TH; ++i) {
      const int64_t t = t0 + half * TH + i;
      if (t < T) ssq[(int64_t)s * T + t] = sq[i];
    }
  }
}

// fp32 MFMA router GEMM for many tokens and E <= 128 experts (E a multiple of 4,
// D of 32, x and G 16-byte aligned): part[s][t][e]
// over the s-th slice of d.  A workgroup owns 32 tokens x 128 experts of one
// slice; x and G pass through LDS in 32-row chunks (two chunks in flight ahead
// of the multiplies).  Wavefront w takes tokens 16*(w&1) .. +15 and experts
// 64*(w>>1) .. +63 as four 16x16 tiles of v_mfma_f32_16x16x4_f32 (fp32 products
// and sums).  Within each 16-row step of a chunk, MFMA j has lane group g
// supply row 4g + j, so every operand read is one conflict-free dword; the four
// MFMAs of a step cover the step's 16 rows.  G stays in the L2 across the
// 32-token tiles of a slice.
constexpr int RT_T = 32, RT_E = 128, RT_K = 32;

__global__ __launch_bounds__(256) void router_tiled_kernel(const float* __restrict__ x, int64_t T,
                                                           int D, const float* __restrict__ G,
                                                           int E, int dchunk,
                                                           float* __restrict__ part,
                                                           float* __restrict__ ssq) {
  __shared__ float xs[RT_K][RT_T + 4];        // [row][token], padded
  __shared__ __attribute__((aligned(16))) float gs[RT_K][RT_E];
  constexpr int XL = RT_T * RT_K / 256, GL = RT_K * RT_E / 256;   // loads per thread per chunk
  const int tid = threadIdx.x, lane = tid % WAVE;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int th = wave & 1, eh = wave >> 1;    // token half, expert half
  const int ln = lane % 16, lg = lane / 16;
  const int64_t t0 = (int64_t)blockIdx.x * RT_T;
  const int sl = blockIdx.y;
  const int d0 = sl * dchunk, d1 = min(D, d0 + dchunk);
  f32x4 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sq = 0.f;                             // x^2 over this lane's rows, token 16*th + ln
  // Two register stages of 16-byte loads (clamped addresses, so every load is
  // unconditional; values past the slice or the token range are masked at the LDS
  // store): a 64-row slice costs one memory round trip.
  constexpr int XL4 = XL / 4, GL4 = GL / 4;
  struct Stage {
    float4 x[XL4], g[GL4];
  };
  auto load = [&](int dd, Stage& st) {
#pragma unroll
    for (int j = 0; j < XL4; ++j) {
      const int i = j * 256 + tid, tt = i / (RT_K / 4), c = 4 * (i % (RT_K / 4));
      const int64_t t = min(t0 + tt, T - 1);
      st.x[j] = *(const float4*)(x + t * D + min(dd + c, D - 4));
    }
#pragma unroll
    for (int j = 0; j < GL4; ++j) {
      const int i = j * 256 + tid, c = i / (RT_E / 4), e = 4 * (i % (RT_E / 4));
      st.g[j] = *(const float4*)(G + (int64_t)min(dd + c, D - 1) * E + min(e, E - 4));
    }
  };
  auto store = [&](int dd, const Stage& st) {
#pragma unroll
    for (int j = 0; j < XL4; ++j) {
      const int i = j * 256 + tid, tt = i / (RT_K / 4), c = 4 * (i % (RT_K / 4));
      const bool ok = t0 + tt < T && dd + c < d1;    // d1 - dd is a multiple of 4
      xs[c][tt] = ok ? st.x[j].x : 0.f;
      xs[c + 1][tt] = ok ? st.x[j].y : 0.f;
      xs[c + 2][tt] = ok ? st.x[j].z : 0.f;
      xs[c + 3][tt] = ok ? st.x[j].w : 0.f;
    }
#pragma unroll
    for (int j = 0; j < GL4; ++j) {
      const int i = j * 256 + tid, c = i / (RT_E / 4), e = 4 * (i % (RT_E / 4));
      const bool ok = e < E && dd + c < d1;          // E is a multiple of 4
      *(float4*)&gs[c][e] = ok ? st.g[j] : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto mfma_chunk = [&]() {
#pragma unroll
    for (int kk = 0; kk < RT_K; kk += 16) {
      float a[4], b[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = xs[kk + 4 * lg + j][16 * th + ln];
#pragma unroll
        for (int n = 0; n < 4; ++n) b[n][j] = gs[kk + 4 * lg + j][64 * eh + 16 * n + ln];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sq = fmaf(a[j], a[j], sq);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[n][j], acc[n], 0, 0, 0);
      }
    }
  };
  Stage s0, s1;
  load(d0, s0);
  load(d0 + RT_K, s1);
  for (int dd = d0; dd < d1; dd += 2 * RT_K) {
    store(dd, s0);
    __syncthreads();
    load(dd + 2 * RT_K, s0);
    mfma_chunk();
    __syncthreads();
    if (dd + RT_K >= d1) break;                   // uniform
    store(dd + RT_K, s1);
    __syncthreads();
    load(dd + 3 * RT_K, s1);
    mfma_chunk();
    __syncthreads();
  }
  // the four lane groups hold disjoint rows of token 16*th + ln
  sq += __shfl_xor(sq, 16, WAVE);
  sq += __shfl_xor(sq, 32, WAVE);
  if (ssq && eh == 0 && lg == 0) {
    const int64_t t = t0 + 16 * th + ln;
    if (t < T) ssq[(int64_t)sl * T + t] = sq;
  }
  // lane (ln, lg) holds tokens 4*lg + i of the wave's half, expert ln of tile n
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + 16 * th + 4 * lg + i;
    if (t >= T) continue;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int e = 64 * eh + 16 * n + ln;
      if (e < E) part[((int64_t)sl * T + t) * E + e] = acc[n][i];
    }
  }
}

hipError_t launch_router_partial(const float* x, int64_t T, int D, const float* G, int E,
                                 float* part, int ksplit, hipStream_t s, float* ssq) {
  const int dchunk = router_dchunk(D, ksplit);
  auto a16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
  if (E <= RT_E && T >= RT_T && E % 4 == 0 && D % 32 == 0 && a16(x) && a16(G)) {
    dim3 grid((unsigned)((T + RT_T - 1) / RT_T), (unsigned)ksplit);
    hipLaunchKernelGGL(router_tiled_kernel, grid, dim3(256), 0, s, x, T, D, G, E, dchunk, part, ssq);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((T + 7) / 8), (unsigned)ksplit);
  hipLaunchKernelGGL(router_partial_kernel<8>, grid, dim3(256), 0, s, x, T, D, G, E, dchunk, part,
                     ssq);
  return hipGetLastError();
}

// One wavefront per token: sum the D-slice partials (fixed order), scale by the
// RMSNorm factor when the router saw the raw input, add the bias, pick k
// winners by (value desc, index asc), then weights
// w_j = exp(l_j - l_max) / sum_selected exp(l - l_max), written in ascending id order.
// PL = logits per lane (E <= 64 * PL).
template <int PL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ part, int ksplit,
                                                   int64_t T, int E,
                                                   const float* __restrict__ bias, int k,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w, TopkExtra ex) {
  __shared__ float sel_l[4][MAX_K];
  __shared__ int sel_e[4][MAX_K];
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wavefront leaves together; no block barrier below
  // Common shapes (at most 32 D-slices, E <= 128, D <= 2048): every load of the
  // token -- the per-slice sums of squares, the partial logits and the input
  // row -- is issued before the first wait, so the token costs one memory round
  // trip instead of three.  Indices are clamped, so the loads are unconditional.
  if constexpr (PL <= 2) {
  if (ksplit <= 32 && (!ex.xhi || ex.D <= 8 * 4 * WAVE)) {
    float sv[32], pv[PL][32];
    float4 q[8];
    const float* xr = ex.x + t * ex.D;
    if (ex.ssq) {
#pragma unroll
      for (int j = 0; j < 32; ++j) sv[j] = ex.ssq[(int64_t)min(j, ksplit - 1) * T + t];
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = min(i * WAVE + lane, E - 1);
#pragma unroll
      for (int j = 0; j < 32; ++j) pv[i][j] = part[((int64_t)min(j, ksplit - 1) * T + t) * E + e];
    }
    if (ex.xhi) {
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = *(const float4*)(xr + min(4 * (j * WAVE + lane), ex.D - 4));
    }
    float inv = 1.0f;
    if (ex.ssq) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (j < ksplit) ss += sv[j];
      inv = 1.0f / sqrtf(ss / (float)ex.D + PRENORM_EPS);
      if (ex.inv && lane == 0) ex.inv[t] = inv;
    }
    if (ex.xhi) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = 4 * (j * WAVE + lane);
        if (d >= ex.D) break;
        const float u[4] = {q[j].x * inv, q[j].y * inv, q[j].z * inv, q[j].w * inv};
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = (_Float16)u[i];
          lo[i] = (_Float16)(u[i] - (float)hi[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ex.xhi[t * ex.D + plane_pos(d + i)] = hi[i];
        if (ex.xlo) {
#pragma unroll
          for (int i = 0; i < 4; ++i) ex.xlo[t * ex.D + plane_pos(d + i)] = lo[i];
        }
      }
    }
    float v[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = i * WAVE + lane;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (j < ksplit) sum += pv[i][j];                // slice order, as below
      float l = -FLT_MAX;
      if (e < E) {
        l = sum * inv;
        if (bias) l += bias[e];
      }
      v[i] = l;
    }
    select_and_write<PL>(v, E, k, t, wave, lane, sel_l, sel_e, ids, w);
    return;
  }
  }
  // RMSNorm factor from the router's per-slice sums of squares (slice order)
  float inv = 1.0f;
  if (ex.ssq) {
    float ss = 0.f;
    for (int p0 = 0; p0 < ksplit; p0 += 32) {
      float pv[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) pv[j] = ex.ssq[(int64_t)min(p0 + j, ksplit - 1) * T + t];
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (p0 + j < ksplit) ss += pv[j];
    }
    inv = 1.0f / sqrtf(ss / (float)ex.D + PRENORM_EPS);
    if (ex.inv && lane == 0) ex.inv[t] = inv;
  }
  // fp16 planes of u = inv * x for the MFMA expert kernels (eight float4 loads per
  // lane in flight at a time)
  if (ex.xhi) {
    const float* xr = ex.x + t * ex.D;
    for (int d0 = 0; d0 < ex.D; d0 += 8 * 4 * WAVE) {
      float4 q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = *(const float4*)(xr + min(d0 + 4 * (j * WAVE + lane), ex.D - 4));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = d0 + 4 * (j * WAVE + lane);
        if (d >= ex.D) break;
        const float u[4] = {q[j].x * inv, q[j].y * inv, q[j].z * inv, q[j].w * inv};
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = (_Float16)u[i];
          lo[i] = (_Float16)(u[i] - (float)hi[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ex.xhi[t * ex.D + plane_pos(d + i)] = hi[i];
        if (ex.xlo) {
#pragma unroll
          for (int i = 0; i < 4; ++i) ex.xlo[t * ex.D + plane_pos(d + i)] = lo[i];
        }
      }
    }
  }
  float v[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = i * WAVE + lane;
    float s = -FLT_MAX;
    if (e < E) {
      // 32 partials in flight at a time, summed in slice order
      s = 0.f;
      for (int p0 = 0; p0 < ksplit; p0 += 32) {
        float pv[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int p = min(p0 + j, ksplit - 1);
          pv[j] = part[((int64_t)p * T + t) * E + e];
        }
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (p0 + j < ksplit) s += pv[j];
      }
      s *= inv;
      if (bias) s += bias[e];
    }
    v[i] = s;
  }
  select_and_write<PL>(v, E, k, t, wave, lane, sel_l, sel_e, ids, w);
}

hipError_t launch_topk(const float* part, int ksplit, int64_t T, int E, const float* bias, int k,
                       int32_t* ids, float* w, hipStream_t s, const TopkExtra& ex) {
  static_assert(MAX_E <= 16 * WAVE, "logits per lane");
  dim3 grid((unsigned)((T + 3) / 4));
  if (E <= WAVE)
    hipLaunchKernelGGL(topk_kernel<1>, grid, dim3(256), 0, s, part, ksplit, T, E, bias, k, ids, w, ex);
  else if (E <= 2 * WAVE)
    hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(256), 0, s, part, ksplit, T, E, bias, k, ids, w, ex);
  else if (E <= 4 * WAVE)
    hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, s, part, ksplit, T, E, bias, k, ids, w, ex);
  else
    hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, s, part, ksplit, T, E, bias, k, ids, w, ex);
  return hipGetLastError();
}

}  // namespace moe
