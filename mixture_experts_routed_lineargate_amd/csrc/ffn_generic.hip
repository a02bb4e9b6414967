// Generic routed expert SwiGLU FFN kernels: any D, F that are multiples of 32,
// either block format, any alignment of even bases.  One workgroup per
// (flat row r = t*k + j, output chunk); weights are read once per row, so
// these serve shapes the tuned kernels do not cover and the small toy layer.
//
// Each wavefront computes one output at a time: lanes 0-31 take element i of
// block b, lanes 32-63 element i of block b+1, so a wave reads 68 (Q8_0) or
// 36 (Q4) contiguous bytes per step and the activation reads from LDS are
// conflict-free.  Block value = fp16 scale * q (Q8_0) or scale * (q - 8) (Q4),
// exact in fp32; products are accumulated in fp32.
#include "internal.hpp"

namespace moe {

__device__ inline float row_dot_generic(const uint8_t* __restrict__ row, int nb,
                                        const float* __restrict__ xs, int fmt) {
  const int lane = threadIdx.x % WAVE;
  const int sub = lane >> 5, i = lane & 31;
  float acc = 0.f;
  if (fmt == MOE_FMT_Q8_0) {
    for (int b = sub; b < nb; b += 2) {
      const uint8_t* blk = row + (int64_t)b * 34;
      const float d = half_bits_to_float(*(const uint16_t*)blk);
      const float q = (float)(int8_t)blk[2 + i];
      acc = fmaf(d * q, xs[b * QK + i], acc);
    }
  } else {
    for (int b = sub; b < nb; b += 2) {
      const uint8_t* blk = row + (int64_t)b * 18;
      const float d = half_bits_to_float(*(const uint16_t*)blk);
      const uint32_t byte = blk[2 + (i >> 1)];
      const int q = (int)((i & 1) ? (byte >> 4) : (byte & 15u)) - 8;
      acc = fmaf(d * (float)q, xs[b * QK + i], acc);
    }
  }
  return wave_sum(acc);
}

constexpr int GEN_CHUNK = 64;  // outputs per workgroup

__global__ __launch_bounds__(256) void gateup_generic_kernel(const float* __restrict__ x,
                                                             ExpertsDev W,
                                                             const int32_t* __restrict__ ids,
                                                             int64_t T, int k,
                                                             float* __restrict__ h) {
  extern __shared__ float xs[];
  const int64_t r = blockIdx.x;
  const int64_t t = r / k;
  const int e = ids[r];
  const int D = W.D, F = W.F;
  const int f0 = blockIdx.y * GEN_CHUNK;
  const int f1 = min(F, f0 + GEN_CHUNK);
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  if ((unsigned)e >= (unsigned)W.E) {
    for (int f = f0 + threadIdx.x; f < f1; f += blockDim.x) h[r * F + f] = 0.f;
    return;
  }
  for (int d = threadIdx.x; d < D; d += blockDim.x) xs[d] = x[t * D + d];
  __syncthreads();
  const int64_t rb = (int64_t)(D / QK) * block_bytes(W.fmt);
  const uint8_t* g = W.gate + (int64_t)e * W.gate_stride;
  const uint8_t* u = W.up + (int64_t)e * W.up_stride;
  for (int f = f0 + wave; f < f1; f += blockDim.x / WAVE) {
    const float gv = row_dot_generic(g + f * rb, D / QK, xs, W.fmt);
    const float uv = row_dot_generic(u + f * rb, D / QK, xs, W.fmt);
    if (lane == 0) h[r * F + f] = silu(gv) * uv;
  }
}

__global__ __launch_bounds__(256) void down_generic_kernel(const float* __restrict__ h,
                                                           ExpertsDev W,
                                                           const int32_t* __restrict__ ids,
                                                           int64_t T, int k,
                                                           float* __restrict__ y) {
  extern __shared__ float hs[];
  const int64_t r = blockIdx.x;
  const int e = ids[r];
  const int D = W.D, F = W.F;
  const int d0 = blockIdx.y * GEN_CHUNK;
  const int d1 = min(D, d0 + GEN_CHUNK);
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  if ((unsigned)e >= (unsigned)W.E) {
    for (int d = d0 + threadIdx.x; d < d1; d += blockDim.x) y[r * D + d] = 0.f;
    return;
  }
  for (int f = threadIdx.x; f < F; f += blockDim.x) hs[f] = h[r * F + f];
  __syncthreads();
  const int64_t rb = (int64_t)(F / QK) * block_bytes(W.fmt);
  const uint8_t* dn = W.down + (int64_t)e * W.down_stride;
  for (int d = d0 + wave; d < d1; d += blockDim.x / WAVE) {
    const float v = row_dot_generic(dn + d * rb, F / QK, hs, W.fmt);
    if (lane == 0) y[r * D + d] = v;
  }
}

hipError_t launch_gateup_generic(const float* x, const ExpertsDev& W, const int32_t* ids, int64_t T,
                                 int k, float* h, hipStream_t s) {
  dim3 grid((unsigned)(T * k), (unsigned)((W.F + GEN_CHUNK - 1) / GEN_CHUNK));
  hipLaunchKernelGGL(gateup_generic_kernel, grid, dim3(256), (size_t)W.D * sizeof(float), s, x, W,
                     ids, T, k, h);
  return hipGetLastError();
}

hipError_t launch_down_generic(const float* h, const ExpertsDev& W, const int32_t* ids, int64_t T,
                               int k, float* y, hipStream_t s) {
  dim3 grid((unsigned)(T * k), (unsigned)((W.D + GEN_CHUNK - 1) / GEN_CHUNK));
  hipLaunchKernelGGL(down_generic_kernel, grid, dim3(256), (size_t)W.F * sizeof(float), s, h, W,
                     ids, T, k, y);
  return hipGetLastError();
}

// out[t][d] = sum_j w[t][j] * y[t*k+j][d] (j ascending) (+ residual[t][d]).
// Four outputs per thread when every row is 16-byte aligned (D % 4 == 0 and
// aligned bases), one otherwise; the summation order is the same either way.
// With ids, a slot whose expert id is outside [0, E) was dropped by the
// grouping: its y row was never computed, so it is skipped, and when y_out is
// given its row there is set to zero (the value the header promises for a
// dropped entry).  With k <= KC every load a thread needs (ids, weights, the
// k y rows, the residual) is issued before the first is used: one memory round
// trip instead of one or two per slot.
constexpr int CT = 64;                                 // threads per combine workgroup
constexpr int KC = 8;                                  // slots loaded up front

template <int V>
__global__ __launch_bounds__(CT) void combine_kernel(const float* __restrict__ y,
                                                     const float* __restrict__ w,
                                                     const int32_t* __restrict__ ids, int E,
                                                     float* __restrict__ y_out, int64_t T,
                                                     int k, int D,
                                                     const float* __restrict__ residual,
                                                     const float* __restrict__ res_scale,
                                                     float* __restrict__ out) {
  typedef float fv __attribute__((ext_vector_type(V)));
  const int64_t t = blockIdx.x;
  const int d = (blockIdx.y * CT + threadIdx.x) * V;
  if (d >= D) return;
  auto ld = [&](const float* a) { return *(const fv*)a; };
  fv s = {};
  if (k <= KC) {
    int id[KC];
    float wv[KC];
    fv yv[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const int64_t r = t * k + min(j, k - 1);        // clamped: rows of this token
      id[j] = ids ? ids[r] : 0;
      wv[j] = w[r];
      yv[j] = ld(y + r * D + d);                      // a dropped slot's row: read, not used
    }
    fv rv = {};
    if (residual) rv = ld(residual + t * D + d);
    const float rs = (residual && res_scale) ? res_scale[t] : 1.0f;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      if (j >= k) break;
      if (ids && (unsigned)id[j] >= (unsigned)E) {
        if (y_out) *(fv*)(y_out + (t * k + j) * D + d) = fv{};
        continue;
      }
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] = fmaf(wv[j], yv[j][i], s[i]);
    }
    if (residual) {
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] += res_scale ? rv[i] * rs : rv[i];
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int64_t r = t * k + j;
      if (ids && (unsigned)ids[r] >= (unsigned)E) {
        if (y_out) *(fv*)(y_out + r * D + d) = fv{};
        continue;
      }
      const float wj = w[r];
      const fv v = ld(y + r * D + d);
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] = fmaf(wj, v[i], s[i]);
    }
    if (residual) {
      const float rs = res_scale ? res_scale[t] : 1.0f;   // residual = rs * residual row
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] += res_scale ? residual[t * D + d + i] * rs : residual[t * D + d + i];
    }
  }
  *(fv*)(out + t * D + d) = s;
}

hipError_t launch_combine(const float* y, const float* w, int64_t T, int k, int D,
                          const float* residual, float* out, hipStream_t s,
                          const float* res_scale, const int32_t* ids, int E, float* y_out) {
  auto a16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15) == 0; };
  if (D % 4 == 0 && a16(y) && a16(out) && a16(residual) && a16(y_out)) {
    dim3 grid((unsigned)T, (unsigned)((D / 4 + CT - 1) / CT));
    hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(CT), 0, s, y, w, ids, E, y_out, T, k, D,
                       residual, res_scale, out);
  } else {
    dim3 grid((unsigned)T, (unsigned)((D + CT - 1) / CT));
    hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(CT), 0, s, y, w, ids, E, y_out, T, k, D,
                       residual, res_scale, out);
  }
  return hipGetLastError();
}

// y[r] = 0 for every flat row r whose expert id is outside [0, E) (rows the
// grouping dropped, which the grouped kernels never write).
__global__ __launch_bounds__(256) void zero_dropped_kernel(const int32_t* __restrict__ ids,
                                                           int64_t R, int E, int D,
                                                           float* __restrict__ y) {
  const int64_t r = blockIdx.x;
  if ((unsigned)ids[r] < (unsigned)E) return;
  for (int d = threadIdx.x; d < D; d += 256) y[r * D + d] = 0.f;
}

hipError_t launch_zero_dropped(const int32_t* ids, int64_t R, int E, int D, float* y,
                               hipStream_t s) {
  hipLaunchKernelGGL(zero_dropped_kernel, dim3((unsigned)R), dim3(256), 0, s, ids, R, E, D, y);
  return hipGetLastError();
}

// out[t] = x[t] / sqrt(mean(x[t]^2) + eps); one workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int D,
                                                      float eps, float* __restrict__ out) {
  __shared__ float part[256 / WAVE];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * D;
  float ss = 0.f;
  for (int d = threadIdx.x; d < D; d += 256) ss = fmaf(xr[d], xr[d], ss);
  ss = wave_sum(ss);
  if (threadIdx.x % WAVE == 0) part[threadIdx.x / WAVE] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)D + eps);
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += 256) out[t * D + d] = xr[d] * inv;
}

hipError_t launch_rmsnorm(const float* x, int64_t T, int D, float eps, float* out, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)T), dim3(256), 0, s, x, D, eps, out);
  return hipGetLastError();
}

}  // namespace moe
