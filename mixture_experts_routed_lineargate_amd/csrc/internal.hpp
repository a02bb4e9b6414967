// Internal declarations shared by the HIP translation units of libmoe_mi355x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int QK = 32;          // weights per block
constexpr int WAVE = 64;        // CDNA wavefront
constexpr int MAX_E = 1024;
constexpr int MAX_K = 32;
constexpr float PRENORM_EPS = 1e-6f;

__host__ __device__ inline int block_bytes(int fmt) { return fmt == MOE_FMT_Q8_0 ? 34 : 18; }

// Exact fp16 -> fp32 (subnormals included).
__device__ inline float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

// Device views of one layer's experts.
struct ExpertsDev {
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  int64_t gate_stride, up_stride, down_stride;
  int E, D, F, fmt;
};

inline ExpertsDev to_dev(const moe_experts& w) {
  return ExpertsDev{(const uint8_t*)w.w_gate, (const uint8_t*)w.w_up, (const uint8_t*)w.w_down,
                    w.gate_stride, w.up_stride, w.down_stride,
                    w.num_experts, w.d_model, w.d_ff, w.format};
}

// Workspace carving (all regions 256-byte aligned).
struct Workspace {
  float* part_logits;   // [ksplit][T][E]
  int32_t* ids;         // [T*k]
  float* w;             // [T*k]
  int32_t* offsets;     // [E+1]
  int32_t* rows;        // [T*k]
  float* h;             // [T*k][F]
  float* y;             // [T*k][D]
  float* xn;            // [T][D]  normalised input (PRENORM)
  uint32_t* sync;       // barrier / work-list words
  size_t bytes;
};

int router_ksplit(int64_t T, int D);
Workspace carve_workspace(void* base, int64_t T, int D, int F, int E, int k, int flags);
constexpr size_t SYNC_BYTES = 64 * 1024;

bool trace_enabled();
void trace(const char* what, int64_t T, int D, int F, int E, int k, int fmt);

// ---- launchers (return hipError_t of the launch) ----
hipError_t launch_router_partial(const float* x, int64_t T, int D, const float* G, int E,
                                 float* part, int ksplit, hipStream_t s);
hipError_t launch_topk(const float* part, int ksplit, int64_t T, int E, const float* bias, int k,
                       int32_t* ids, float* w, hipStream_t s);
hipError_t launch_group(const int32_t* ids, int64_t N, int E, int32_t* offsets, int32_t* rows,
                        hipStream_t s);
hipError_t launch_gateup_generic(const float* x, const ExpertsDev& W, const int32_t* ids, int64_t T,
                                 int k, float* h, hipStream_t s);
hipError_t launch_down_generic(const float* h, const ExpertsDev& W, const int32_t* ids, int64_t T,
                               int k, float* y, hipStream_t s);
hipError_t launch_combine(const float* y, const float* w, int64_t T, int k, int D,
                          const float* residual, float* out, hipStream_t s);
hipError_t launch_rmsnorm(const float* x, int64_t T, int D, float eps, float* out, hipStream_t s);

}  // namespace moe
