// Internal declarations shared by the HIP translation units of libmoe_mi355x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Cross-lane reductions on DPP row permutes (a few cycles each) and readlane,
// instead of ds_bpermute shuffles (an LDS round trip each).  All 64 lanes
// must be active.
constexpr int DPP_QUAD_1032 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;      // lane i <-> 15-i within 16 lanes

template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ inline int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ inline float readlane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ inline int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Sum over each group of 8 lanes (every lane of the group gets it).
__device__ inline float sum8(float v) {
  v += dpp<DPP_QUAD_1032>(v);
  v += dpp<DPP_QUAD_2301>(v);
  v += dpp<DPP_ROW_HALF_MIRROR>(v);
  return v;
}

// Sum over the wavefront (every lane gets it).
__device__ inline float wave_sum(float v) {
  v = sum8(v);
  v += dpp<DPP_ROW_MIRROR>(v);
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}

__device__ inline int wave_min(int v) {
  v = min(v, dpp<DPP_QUAD_1032>(v));
  v = min(v, dpp<DPP_QUAD_2301>(v));
  v = min(v, dpp<DPP_ROW_HALF_MIRROR>(v));
  v = min(v, dpp<DPP_ROW_MIRROR>(v));
  return min(min(readlane(v, 0), readlane(v, 16)), min(readlane(v, 32), readlane(v, 48)));
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
  _Float16* xp;         // [2][T][D] fp16 planes of the layer input (grouped kernels)
  float* ssq;           // [ksplit][T] per-slice sums of squares of the layer input
  float* inv;           // [T] RMSNorm factors
  uint32_t* sync;       // barrier / work-list words
  size_t bytes;
};

int router_ksplit(int64_t T, int D);
Workspace carve_workspace(void* base, int64_t T, int D, int F, int E, int k, int flags);
// Activation planes (the fp16 hi / lo rows of x or h that the MFMA expert kernels
// read) hold each group of 8 consecutive values in the order 0, 2, 4, 6, 1, 3, 5, 7:
// the order in which one byte permute per pair rebuilds a block's codes as fp16
// (the low, then the high nibbles of four bytes; the even, then the odd bytes of
// two dwords).  plane_pos(k) is the position of value k in its row.
__host__ __device__ constexpr int plane_pos(int k) {
  return (k & ~7) | ((k & 1) << 2) | ((k & 7) >> 1);
}
static_assert(plane_pos(1) == 4 && plane_pos(2) == 1 && plane_pos(7) == 7 && plane_pos(14) == 11,
              "plane order");

constexpr size_t SYNC_BYTES = 4 * 1024 * 1024;  // barrier words and exchange buffers
constexpr size_t ROUTE_SYNC_OFF = 2 * 1024 * 1024;  // small-batch routing's exchange words
constexpr size_t STACK_ACC_OFF = 1280 * 1024;      // decode stack accumulators (written by no other kernel)
constexpr size_t ERR_WORD_OFF = 64;                 // u32 error word (bounded wait gave up)
constexpr size_t NOALLOC_SCRATCH_BYTES = 8u << 20;  // moe_layer_noalloc's static workspace

bool trace_enabled();
void trace(const char* what, int64_t T, int D, int F, int E, int k, int fmt);

// ---- launchers (return hipError_t of the launch) ----
// ssq (optional, [ksplit][T]): each slice's per-token sum of x^2 as well
hipError_t launch_router_partial(const float* x, int64_t T, int D, const float* G, int E,
                                 float* part, int ksplit, hipStream_t s, float* ssq = nullptr);
// With ssq: inv_t = 1/sqrt(mean(x_t^2) + eps) scales the logits (the router is
// linear in x) and goes to inv[t]; with xhi: the fp16 planes of u_t = inv_t x_t
// (inv_t = 1 without ssq) go to xhi / xlo (xlo may be null).
struct TopkExtra {
  const float* ssq = nullptr;
  int D = 0;
  float* inv = nullptr;
  const float* x = nullptr;
  _Float16* xhi = nullptr;
  _Float16* xlo = nullptr;
};
hipError_t launch_topk(const float* part, int ksplit, int64_t T, int E, const float* bias, int k,
                       int32_t* ids, float* w, hipStream_t s, const TopkExtra& ex = TopkExtra());
// Router + top-k (+ RMSNorm factor and input planes) + grouping of at most 32
// tokens in one launch (route_small.hip).
bool route_small_supported(int64_t T, int D, int E, int k);
hipError_t launch_route_small(const float* x, int64_t T, int D, const float* G, const float* bias,
                              int E, int k, bool prenorm, int32_t* ids, float* w, float* inv,
                              _Float16* xhi, _Float16* xlo, int32_t* offsets, int32_t* rows,
                              const Workspace& ws, hipStream_t s);
hipError_t launch_group(const int32_t* ids, int64_t N, int E, int32_t* offsets, int32_t* rows,
                        hipStream_t s);
hipError_t launch_gateup_generic(const float* x, const ExpertsDev& W, const int32_t* ids, int64_t T,
                                 int k, float* h, hipStream_t s);
hipError_t launch_down_generic(const float* h, const ExpertsDev& W, const int32_t* ids, int64_t T,
                               int k, float* y, hipStream_t s);
// residual row t is scaled by res_scale[t] when res_scale is given; with ids,
// slots whose id is outside [0, E) are skipped (and their y_out rows zeroed)
hipError_t launch_combine(const float* y, const float* w, int64_t T, int k, int D,
                          const float* residual, float* out, hipStream_t s,
                          const float* res_scale = nullptr, const int32_t* ids = nullptr,
                          int E = 0, float* y_out = nullptr);
// y rows of dropped entries (expert id outside [0, E)) set to zero
hipError_t launch_zero_dropped(const int32_t* ids, int64_t R, int E, int D, float* y,
                               hipStream_t s);
hipError_t launch_rmsnorm(const float* x, int64_t T, int D, float eps, float* out, hipStream_t s);

// grouped GEMM on MFMA (batched / prefill expert FFN)
enum { GG_A_TOKEN = 0, GG_A_FLAT = 1, GG_A_SORTED = 2 };   // activation row of sorted row i:
                                                          // x[rows[i]/k], h[rows[i]], h[i]
bool grouped_supported(const ExpertsDev& W, bool need_gate_up);
bool grouped_fits(int64_t T, int64_t R, const ExpertsDev& W);
hipError_t launch_grouped_gateup(const _Float16* xhi, const _Float16* xlo, int a_mode,
                                 const ExpertsDev& W, const int32_t* offsets, const int32_t* rows,
                                 int64_t R, int k, _Float16* hhi, _Float16* hlo, bool split,
                                 hipStream_t s);
hipError_t launch_grouped_down(const _Float16* hhi, const _Float16* hlo, int a_mode,
                               const ExpertsDev& W, const int32_t* offsets, const int32_t* rows,
                               int64_t R, int k, float* y, bool split, hipStream_t s,
                               bool banded = false);
hipError_t launch_to_planes(const float* src, int64_t n, _Float16* hi, _Float16* lo,
                            hipStream_t s);
// few rows per expert (R <= 512) at the tuned geometry: weight-slice kernels, same operands
bool skinny_supported(const ExpertsDev& W, int64_t R, bool need_gate_up);
hipError_t launch_skinny_gateup(const _Float16* xhi, const _Float16* xlo, int a_mode,
                                const ExpertsDev& W, const int32_t* offsets, const int32_t* rows,
                                int64_t R, int k, _Float16* hhi, _Float16* hlo, bool split,
                                hipStream_t s);
hipError_t launch_skinny_down(const _Float16* hhi, const _Float16* hlo, int a_mode,
                              const ExpertsDev& W, const int32_t* offsets, const int32_t* rows,
                              int64_t R, int k, float* y, bool split, hipStream_t s);

// single-token decode through one layer or a stack of layers in one launch
// (D 2048, F 768, E 128, k 8)
struct StackLayer {
  const float* gate;
  const float* bias;
  ExpertsDev W;
};
int decode_stack_max_layers();
// one layer's pointers and the token's fit the fused kernel (geometry, alignment,
// all workgroups resident)
bool decode_stack_layer_ok(const ExpertsDev& W, int k);
bool decode_stack_io_ok(const float* x, const float* out);
hipError_t launch_decode_stack(const float* x, int L, const StackLayer* layers, int fmt,
                               bool prenorm0, bool residual, float* outs, int32_t* ids, float* w,
                               int32_t* offsets, int32_t* rows, const Workspace& ws,
                               hipStream_t s);

// attention-side primitives (attn_prep.hip); ws: 256 header bytes (error word at 64),
// [T][N] tagged 64-bit published rows, then (at attn_count_offset) [ceil(T/8)][Hq + Hkv]
// u32 ticket counters; zero-filled before first use
size_t attn_lds_bytes(int D, int fmt);
size_t attn_count_offset(int64_t T, int N);
hipError_t launch_attn_prep(const float* x, int64_t T, int D, const float* attn_gain,
                            const uint8_t* w_qkv, int fmt, int Hq, int Hkv, int hd,
                            const float* q_gain, const float* k_gain, const int32_t* pos,
                            float theta, float eps, float* q, float* k_cache, float* v_cache,
                            int max_pos, void* ws, hipStream_t s);

}  // namespace moe
