// Fused single-token decode layer for the Qwen3-MoE geometry (d_model 2048,
// d_ff 768, 128 experts, top-8; evidence page, Model card): router -> top-8 ->
// gate/up + SwiGLU -> down + weighted combine (+ residual) in ONE launch, so
// the warm path has no host synchronisation and no launch gaps between its
// steps (evidence page: fewer warm host synchronisations; technical-overview
// page: warm target path router -> resident expert -> combine).
//
// 256 workgroups of 512 threads, one per CU.  Workgroup w owns expert slot
// j = w / 32 and part r = w % 32 of that expert:
//  phase 1  workgroups 0..63 form an 8 x 8 grid over (16 experts, 256 rows of
//           the 2048x128 gate) and publish partial logits; they also write
//           the initial value of 32 outputs (the residual, or 0).
//  phase 2  every workgroup gathers the 8 partials of each logit, adds the
//           bias, picks the top-8 by rank counting over the whole workgroup
//           (lower index wins ties) and their weights.
//  phase 3  it loads its whole weight share at once: 24 gate rows + 24 up rows
//           of expert j (f = 24r..24r+23) and 64 down rows (d = 64r..64r+63),
//           ~153 KB for Q8_0, into registers; writes gate/up to LDS, computes
//           h_j(f) = silu(g)*u for its 24 rows and publishes them.
//  phase 4  it gathers h_j (768 values), finishes y_j(d) for its 64 rows from
//           the down rows in LDS and adds w_j y_j(d) into out(d) with an fp32
//           atomic (or, with MOE_F_DETERMINISTIC, publishes w_j y_j(d) and
//  phase 5  the owner of each output sums the 8 expert terms in slot order).
//
// The exchange protocol, the register dequant and the top-8 selection are
// shared with the multi-layer kernel (decode_common.hpp).
#include "decode_common.hpp"

namespace moe {
namespace dec {

struct Args {
  const float* x;
  const float* gate;
  const float* bias;
  ExpertsDev W;
  float* out;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* offsets;
  int32_t* rows;
  uint64_t* part;     // [PREP][RDS][E] tagged partial logits
  uint64_t* h;        // [HREP][K][F] tagged h
  uint64_t* y;        // [K][D]   tagged weighted expert outputs (deterministic combine)
  uint32_t* epochs;   // [NWG]    launch counters
  uint32_t* err;      // poll timeout flag
  int flags;
};

template <int FMT>
__global__ __launch_bounds__(NT, 1) void decode_layer_kernel(Args p) {
  using G = Geo<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES + 16];  // +16: reads may pass a row end by 2 bytes
  __shared__ float red[NT];
  __shared__ float rsum[REPG];
  __shared__ __attribute__((aligned(16))) float lg[E];
  __shared__ __align__(16) int top[K];
  __shared__ int sel_e[K];
  __shared__ float sel_w[K];

  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int wg = blockIdx.x;
  const int slot = wg / PARTS, part = wg % PARTS;
  const bool deterministic = (p.flags & MOE_F_DETERMINISTIC) != 0;
  const bool router = wg < RW;
  float* xs = (float*)lds;   // the input row [D]; aliases the gate/up region, free until phase 3

  // ---- issue every load that depends on nothing: x, this workgroup's gate rows, the epoch ----
  // Router workgroup (eg, ds) multiplies rows 256*ds..+255 of the gate by x for
  // experts 16*eg..+15; thread (rg, el) takes 8 rows of expert el.
  // Every workgroup issues the gate loads (the others re-read a router workgroup's rows
  // from the L2 and drop them): conditional loads would make the wait for x also wait
  // for them.
  const float4 xq = ((const float4*)p.x)[tid];
  const int eg = (wg % RW) % REG, ds = (wg % RW) / REG;
  const int el = tid % REPG, rg = tid / REPG;
  const int d0 = ds * (D / RDS) + rg * RROWS;
  float gq[RROWS];
#pragma unroll
  for (int r = 0; r < RROWS; ++r) gq[r] = p.gate[(int64_t)(d0 + r) * E + eg * REPG + el];
  const uint32_t epoch =
      __hip_atomic_load(p.epochs + wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  uint32_t budget = SPIN_LIMIT;

  // ---- input scaling (RMSNorm transition when PRENORM) ----
  ((float4*)xs)[tid] = xq;
  float inv = 1.f;
  if (p.flags & MOE_F_PRENORM) {
    float ss = xq.x * xq.x + xq.y * xq.y + xq.z * xq.z + xq.w * xq.w;
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) tot += red[w];
    inv = 1.0f / sqrtf(tot / (float)D + PRENORM_EPS);
  }
  __syncthreads();                                  // xs complete; red free again

  // initial value of 8 outputs for the atomic combine, issued as early as possible
  if (router && !deterministic && tid < D / RW) {
    const int d = wg * (D / RW) + tid;
    const float init = (p.flags & MOE_F_RESIDUAL) ? xs[d] * inv : 0.f;
    __hip_atomic_store(p.out + d, init, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // x (scaled by the RMSNorm factor) as digit planes (all threads, LDS past xs),
  // then this lane's block (block `lane` of the 2048-wide input) into registers
  uint8_t* xdig = lds + D * 4;
  float2* xscl = (float2*)(lds + D * 4 + (D / QK) * 96);
  act_digits_lds<FMT, 4>(xs, inv, D / QK, xdig, xscl);
  __syncthreads();
  ActDig xd;
  load_dig(xdig, xscl, lane, xd);

  // ---- phase 1: partial router logits (x is scaled by the RMSNorm factor afterwards) ----
  if (router) {
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < RROWS; ++r) acc = fmaf(xs[d0 + r], gq[r], acc);
    red[tid] = acc;
    __syncthreads();
    if (tid < REPG) {
      float sum = 0.f;
      for (int g = 0; g < RGRP; ++g) sum += red[g * REPG + tid];
      rsum[tid] = sum * inv;
    }
    // the output initialisation must land before any partial of this workgroup is
    // visible (it was issued long before, so this wait is short)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    {
      const int rep = tid / REPG;
      publish(p.part + (rep * RDS + ds) * E + eg * REPG + el, epoch, rsum[el]);
    }
  }

  // ---- phase 2: logits, top-8, weights (wavefront 0) ----
  if (wave == 0) {
    float pv[2 * RDS];
    const uint64_t* rep = p.part + (wg % PREP) * RDS * E;
    gather<2 * RDS>(rep + lane, WAVE, epoch, p.err, budget, pv);     // [ds][e], e = lane, lane + 64
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int ds = 0; ds < RDS; ++ds) {
      v0 += pv[2 * ds];
      v1 += pv[2 * ds + 1];
    }
    if (p.bias) {
      v0 += p.bias[lane];
      v1 += p.bias[lane + WAVE];
    }
    lg[lane] = v0;
    lg[lane + WAVE] = v1;
    if (lane < K) top[lane] = -1;
  }
  __syncthreads();
  select_top8_block(lg, top, sel_e, sel_w);

  // ---- phase 3: load this workgroup's whole weight share ----
  const int e_j = min(max(sel_e[slot], 0), E - 1);
  const int f0 = part * FPW;
  const int dr0 = part * DPW;
  const uint8_t* gsrc = p.W.gate + (int64_t)e_j * p.W.gate_stride + (int64_t)f0 * G::GU_ROW;
  const uint8_t* usrc = p.W.up + (int64_t)e_j * p.W.up_stride + (int64_t)f0 * G::GU_ROW;
  const uint8_t* dsrc = p.W.down + (int64_t)e_j * p.W.down_stride + (int64_t)dr0 * G::DN_ROW;

  u32x4 gu[G::NGRP][G::GRP_ITERS];
  u32x4 dn[G::DN_ITERS];
#pragma unroll
  for (int g = 0; g < G::NGRP; ++g) {
#pragma unroll
    for (int it = 0; it < G::GRP_ITERS; ++it) {
      // unconditional (clamped) loads keep the compiler's wait counts exact
      const int c = min(it * NT + tid, G::GRP_CHUNKS - 1);
      constexpr int half = G::GRP_CHUNKS / 2;         // gate rows first, then up rows
      const int64_t row_off = (int64_t)(g * G::PPG) * G::GU_ROW;
      const uint8_t* src = c < half ? gsrc + row_off + 16 * c : usrc + row_off + 16 * (c - half);
      gu[g][it] = __builtin_nontemporal_load((const u32x4*)src);
    }
  }
#pragma unroll
  for (int it = 0; it < G::DN_ITERS; ++it) {
    const int c = min(it * NT + tid, G::DN_CHUNKS - 1);
    dn[it] = __builtin_nontemporal_load((const u32x4*)(dsrc + 16 * c));
  }
#pragma unroll
  for (int g = 0; g < G::NGRP; ++g) {
#pragma unroll
    for (int it = 0; it < G::GRP_ITERS; ++it) {
      const int c = it * NT + tid;
      if (c < G::GRP_CHUNKS) *(u32x4*)(lds + g * G::GRP_BYTES + 16 * c) = gu[g][it];
    }
    __syncthreads();
    // wavefront w computes the (gate, up) pair w of this group
    const uint32_t gbase = g * G::GRP_BYTES + wave * G::GU_ROW + lane * G::BB;
    const float gv = wave_sum(block_dot_dig<FMT>(lds, gbase, xd));
    const float uv = wave_sum(block_dot_dig<FMT>(lds, gbase + G::PPG * G::GU_ROW, xd));
    if (lane < HREP)
      publish(p.h + (lane * K + slot) * F + f0 + g * G::PPG + wave, epoch, silu(gv) * uv);
  }
#pragma unroll
  for (int it = 0; it < G::DN_ITERS; ++it) {
    const int c = it * NT + tid;
    if (c < G::DN_CHUNKS) *(u32x4*)(lds + G::DN_OFF + 16 * c) = dn[it];
  }

  // ---- phase 4: y_j for 64 down rows ----
  __syncthreads();                                  // every wave is done with the gate/up region
  float* hs = (float*)lds;                          // h_j [F], reuses the gate/up region
  if (tid < F / 2) {
    float hv2[2];
    gather<2>(p.h + ((part % HREP) * K + slot) * F + tid, F / 2, epoch, p.err, budget, hv2);
    hs[tid] = hv2[0];
    hs[tid + F / 2] = hv2[1];
  }
  __syncthreads();
  // h_j as digit planes, 24 blocks (free gate/up region past h)
  uint8_t* hdig = lds + 4096;
  float2* hscl = (float2*)(lds + 4096 + (F / QK) * 96);
  act_digits_lds<FMT, 2>(hs, 1.0f, F / QK, hdig, hscl);
  __syncthreads();
  {
    const int rl = lane >> 3, sub = lane & 7;       // 8 rows per wavefront, 8 lanes per row
    const int row = wave * 8 + rl;                  // 0..63
    float acc = 0.f;
#pragma unroll
    for (int bi = 0; bi < 3; ++bi) {
      const int b = sub + 8 * bi;                   // 24 blocks per down row
      ActDig hd;
      load_dig(hdig, hscl, b, hd);
      acc += block_dot_dig<FMT>(lds, G::DN_OFF + row * G::DN_ROW + b * G::BB, hd);
    }
    acc = sum8(acc);
    if (sub == 0) {
      const int d = dr0 + row;
      const float v = sel_w[slot] * acc;
      if (deterministic)
        publish(p.y + slot * D + d, epoch, v);
      else
        __hip_atomic_fetch_add(p.out + d, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- phase 5 (deterministic combine): out(d) = sum_j w_j y_j(d) in slot order ----
  if (deterministic && tid < OPW) {
    const int d = wg * OPW + tid;
    float yv[K];
    gather<K>(p.y + d, D, epoch, p.err, budget, yv);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) s += yv[j];
    if (p.flags & MOE_F_RESIDUAL) s += p.x[d] * inv;
    p.out[d] = s;
  }

  // ---- optional routing outputs (workgroup 0) ----
  if (wg == 0) {
    if (p.topk_ids && tid < K) p.topk_ids[tid] = sel_e[tid];
    if (p.topk_w && tid < K) p.topk_w[tid] = sel_w[tid];
    if (p.rows && tid < K) p.rows[tid] = tid;
    if (p.offsets && tid <= E) {
      int c = 0;
#pragma unroll
      for (int r = 0; r < K; ++r) c += sel_e[r] < tid;
      p.offsets[tid] = c;
    }
  }
  if (tid == 0)
    __hip_atomic_store(p.epochs + wg, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT>
static bool fits(int dev) {
  static int cache[64][2];
  if (dev < 0 || dev >= 64) return false;
  int& c = cache[dev][FMT];
  if (c == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_layer_kernel<FMT>, NT, 0) !=
            hipSuccess) {
      c = -1;
    } else {
      c = (cus * per >= NWG) ? 1 : -1;
    }
  }
  return c == 1;
}

}  // namespace dec

bool decode_fused_supported(const ExpertsDev& W, int64_t T, int k, const float* x) {
  if (T != 1 || k != dec::K || W.D != dec::D || W.F != dec::F || W.E != dec::E) return false;
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!a16(x) || !a16(W.gate) || !a16(W.up) || !a16(W.down) || (W.gate_stride & 15) ||
      (W.up_stride & 15) || (W.down_stride & 15))
    return false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  return W.fmt == MOE_FMT_Q8_0 ? dec::fits<MOE_FMT_Q8_0>(dev) : dec::fits<MOE_FMT_Q4>(dev);
}

hipError_t launch_decode_fused(const float* x, const float* gate, const float* bias,
                               const ExpertsDev& W, float* out, int32_t* ids, float* w,
                               int32_t* offsets, int32_t* rows, int flags, const Workspace& ws,
                               hipStream_t s) {
  dec::Args a;
  a.x = x;
  a.gate = gate;
  a.bias = bias;
  a.W = W;
  a.out = out;
  a.topk_ids = ids;
  a.topk_w = w;
  a.offsets = offsets;
  a.rows = rows;
  // exchange buffers live in the workspace's sync region
  char* sync = (char*)ws.sync;
  a.err = ws.sync + ERR_WORD_OFF / sizeof(uint32_t);
  a.epochs = (uint32_t*)(sync + 4096);                    // [256] u32
  a.part = (uint64_t*)(sync + 65536);                     // [32][8][128] u64 (256 KiB)
  a.h = (uint64_t*)(sync + 327680);                       // [4][8][768] u64 (192 KiB)
  a.y = (uint64_t*)(sync + 524288);                       // [8][2048] u64 (128 KiB)
  a.flags = flags;
  if (W.fmt == MOE_FMT_Q8_0)
    hipLaunchKernelGGL(dec::decode_layer_kernel<MOE_FMT_Q8_0>, dim3(dec::NWG), dim3(dec::NT), 0, s, a);
  else
    hipLaunchKernelGGL(dec::decode_layer_kernel<MOE_FMT_Q4>, dim3(dec::NWG), dim3(dec::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
