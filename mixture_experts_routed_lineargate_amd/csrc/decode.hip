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
//           bias, picks the top-8 (one wavefront; lower index wins ties) and
//           their weights.
//  phase 3  it loads its whole weight share at once: 24 gate rows + 24 up rows
//           of expert j (f = 24r..24r+23) and 64 down rows (d = 64r..64r+63),
//           ~153 KB for Q8_0, into registers; writes gate/up to LDS, computes
//           h_j(f) = silu(g)*u for its 24 rows and publishes them.
//  phase 4  it gathers h_j (768 values), finishes y_j(d) for its 64 rows from
//           the down rows in LDS and adds w_j y_j(d) into out(d) with an fp32
//           atomic (or, with MOE_F_DETERMINISTIC, publishes w_j y_j(d) and
//  phase 5  the owner of each output sums the 8 expert terms in slot order).
//
// Exchange between workgroups: every published value is a 64-bit word
// (epoch << 32 | fp32 bits) written with an agent-scope store and read with
// agent-scope loads, which on gfx950 bypass the per-XCD L2, so consumers poll
// the data itself and no grid barrier or L2-wide writeback/invalidate is
// needed.  The epoch is a per-workgroup launch counter kept in the workspace
// (all workgroups run every launch, so their counters agree; the workspace
// must be zero when first used).  Polls are bounded: after ~2^20 rounds a
// workgroup records an error flag and carries on, so a launch always ends.
//
// Dequant in registers: lane b of a wavefront owns block b of a 2048-wide row
// (64 blocks = 64 lanes).  The 34-byte (Q8_0) or 18-byte (Q4) block is read as
// 4-byte-aligned dwords from LDS and realigned with v_alignbyte; int8 codes are
// biased to unsigned (xor 0x80) so one v_cvt_f32_ubyte converts a byte, and
// the bias is removed with the block's activation sum:
//   sum_i q_i x_i = sum_i (q_i + 128) x_i - 128 sum_i x_i   (Q8_0)
//   sum_i (q_i - 8) x_i = sum_i q_i x_i - 8 sum_i x_i        (Q4)
// then multiplied by the fp16 block scale.  Accumulation is fp32.
#include "internal.hpp"

namespace moe {
namespace dec {

constexpr int D = 2048, F = 768, E = 128, K = 8;
constexpr int NWG = 256;             // workgroups
constexpr int NT = 512;              // threads per workgroup
constexpr int NWAVE = NT / WAVE;     // 8
constexpr int PARTS = NWG / K;       // workgroups per expert slot (32)
constexpr int FPW = F / PARTS;       // gate/up rows per workgroup (24)
constexpr int DPW = D / PARTS;       // down rows per workgroup (64)
constexpr int OPW = D / NWG;         // outputs finished per workgroup in phase 5 (8)
constexpr int REG = 8, RDS = 8;      // router grid: expert groups x row slices
constexpr int RW = REG * RDS;        // router workgroups (64)
constexpr int REPG = E / REG;        // experts per router workgroup (16)
constexpr int RGRP = NT / REPG;      // row groups per router workgroup (32)
constexpr int RROWS = D / RDS / RGRP;  // gate rows per thread (8)
constexpr int PREP = 32;             // replicas of the partial logits
constexpr int HREP = 4;              // replicas of h
static_assert(FPW * PARTS == F && DPW * PARTS == D, "split");
static_assert(D / QK == WAVE, "one block per lane for gate/up rows");
static_assert(D % RW == 0 && D / RW <= NT, "router workgroups initialise D / RW outputs each");
static_assert(PREP * REPG == NT, "one replica store per thread");
// Published values are replicated so that no cache line is polled by more than
// 8 workgroups: coherent reads of one line from hundreds of CUs serialise.

template <int FMT>
struct Geo {
  static constexpr int BB = FMT == MOE_FMT_Q8_0 ? 34 : 18;
  static constexpr int GU_ROW = D / QK * BB;          // 2176 / 1152
  static constexpr int DN_ROW = F / QK * BB;          // 816 / 432
  static constexpr int GU_BYTES = FPW * GU_ROW;       // per matrix
  static constexpr int DN_BYTES = DPW * DN_ROW;
  static constexpr int DN_OFF = 2 * GU_BYTES;
  static constexpr int LDS_BYTES = DN_OFF + DN_BYTES;
  // gate/up rows arrive in NGRP groups of PPG (gate, up) row pairs, so the
  // dots of one group overlap the arrival of the next
  static constexpr int NGRP = 3;
  static constexpr int PPG = FPW / NGRP;              // 8 pairs per group
  static constexpr int GRP_BYTES = 2 * PPG * GU_ROW;  // [gate rows][up rows]
  static constexpr int GRP_CHUNKS = GRP_BYTES / 16;
  static constexpr int GRP_ITERS = (GRP_CHUNKS + NT - 1) / NT;
  static constexpr int DN_CHUNKS = DN_BYTES / 16;
  static constexpr int DN_ITERS = (DN_CHUNKS + NT - 1) / NT;
  static_assert(PPG * NGRP == FPW && PPG == NWAVE, "one pair per wavefront per group");
  static_assert(GU_ROW % 16 == 0 && DN_ROW % 16 == 0, "16-byte rows");
  static_assert(LDS_BYTES + 16 + 4096 <= 160 * 1024, "LDS budget");
  static_assert(D * 4 <= 2 * GU_BYTES, "the input row fits in the gate/up region");
  static_assert(F * 4 <= 2 * GU_BYTES, "h staging fits in the gate/up region");
};

constexpr uint32_t SPIN_LIMIT = 1u << 20;

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

__device__ inline uint64_t tag(uint32_t epoch, float v) {
  return ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(v);
}

__device__ inline void publish(uint64_t* p, uint32_t epoch, float v) {
  __hip_atomic_store(p, tag(epoch, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t peek(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until the N tagged words base[i*stride] all carry `epoch` and return
// their values.  All N loads are in flight together; only stragglers are
// polled again.
template <int N>
__device__ inline void gather(const uint64_t* base, int stride, uint32_t epoch, uint32_t* err,
                              float* out) {
  uint64_t v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = peek(base + i * stride);
  for (uint32_t n = 0;; ++n) {
    bool ready = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ready &= (uint32_t)(v[i] >> 32) == epoch;
    if (ready) break;
    if (n == SPIN_LIMIT) {
      __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(4);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((uint32_t)(v[i] >> 32) != epoch) v[i] = peek(base + i * stride);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = __uint_as_float((uint32_t)v[i]);
}

// byte n of v as float (one v_cvt_f32_ubyte<n>)
__device__ inline float ubyte0(uint32_t v) { return (float)(v & 0xffu); }
__device__ inline float ubyte1(uint32_t v) { return (float)((v >> 8) & 0xffu); }
__device__ inline float ubyte2(uint32_t v) { return (float)((v >> 16) & 0xffu); }
__device__ inline float ubyte3(uint32_t v) { return (float)(v >> 24); }

__device__ inline uint32_t lds_u32(const uint8_t* lds, uint32_t byte_off) {
  return *(const uint32_t*)(lds + byte_off);
}

// sum_i w_i x_i for one LDS-resident block (scale applied); xs = sum_i x_i.
template <int FMT>
__device__ inline float block_dot(const uint8_t* lds, uint32_t blk_off, const float* xv, float xs) {
  const uint32_t odd = (blk_off >> 1) & 1u;          // block start is 2 mod 4
  const uint32_t a = blk_off - 2u * odd;              // 4-aligned
  if constexpr (FMT == MOE_FMT_Q8_0) {
    uint32_t dw[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) dw[i] = lds_u32(lds, a + 4u * i);
    const uint32_t sb = odd ? (dw[0] >> 16) : (dw[0] & 0xffffu);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t q = odd ? dw[i + 1] : __builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2);
      q ^= 0x80808080u;
      s = fmaf(ubyte0(q), xv[4 * i + 0], s);
      s = fmaf(ubyte1(q), xv[4 * i + 1], s);
      s = fmaf(ubyte2(q), xv[4 * i + 2], s);
      s = fmaf(ubyte3(q), xv[4 * i + 3], s);
    }
    return half_bits_to_float((uint16_t)sb) * fmaf(-128.f, xs, s);
  } else {
    uint32_t dw[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) dw[i] = lds_u32(lds, a + 4u * i);
    const uint32_t sb = odd ? (dw[0] >> 16) : (dw[0] & 0xffffu);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t n = odd ? dw[i + 1] : __builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2);
      const uint32_t lo = n & 0x0f0f0f0fu, hi = (n >> 4) & 0x0f0f0f0fu;
      // byte j of n holds elements 2j (low nibble) and 2j+1 (high nibble)
      s = fmaf(ubyte0(lo), xv[8 * i + 0], s);
      s = fmaf(ubyte0(hi), xv[8 * i + 1], s);
      s = fmaf(ubyte1(lo), xv[8 * i + 2], s);
      s = fmaf(ubyte1(hi), xv[8 * i + 3], s);
      s = fmaf(ubyte2(lo), xv[8 * i + 4], s);
      s = fmaf(ubyte2(hi), xv[8 * i + 5], s);
      s = fmaf(ubyte3(lo), xv[8 * i + 6], s);
      s = fmaf(ubyte3(hi), xv[8 * i + 7], s);
    }
    return half_bits_to_float((uint16_t)sb) * fmaf(-8.f, xs, s);
  }
}

template <int FMT>
__global__ __launch_bounds__(NT, 1) void decode_layer_kernel(Args p) {
  using G = Geo<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES + 16];  // +16: reads may pass a row end by 2 bytes
  __shared__ float red[NT];
  __shared__ float rsum[REPG];
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

  // this lane's 32 activations (block `lane` of the 2048-wide input)
  float xv[QK];
#pragma unroll
  for (int i = 0; i < QK / 4; ++i) {
    const float4 v = ((const float4*)xs)[lane * (QK / 4) + i];
    xv[4 * i + 0] = v.x * inv;
    xv[4 * i + 1] = v.y * inv;
    xv[4 * i + 2] = v.z * inv;
    xv[4 * i + 3] = v.w * inv;
  }
  float xsum = 0.f;
#pragma unroll
  for (int i = 0; i < QK; ++i) xsum += xv[i];

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
    gather<2 * RDS>(rep + lane, WAVE, epoch, p.err, pv);     // [ds][e], e = lane, lane + 64
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
    uint32_t taken = 0;
    float sl[K];
    int se[K];
#pragma unroll
    for (int r = 0; r < K; ++r) {
      float bv;
      int be;
      const bool ok0 = !(taken & 1u), ok1 = !(taken & 2u);
      if (ok0 && (!ok1 || v0 >= v1)) {
        bv = v0;
        be = lane;
      } else if (ok1) {
        bv = v1;
        be = lane + WAVE;
      } else {
        bv = -3.0e38f;
        be = 0x7fffffff;
      }
      // wave argmax: largest value, then the lowest expert index among equals
      // (a lane's own candidate index is lane or lane + 64)
      const float m = wave_max(bv);
      const uint64_t lo = __ballot(bv == m && be < WAVE);
      const uint64_t any = __ballot(bv == m);
      const int wl = __ffsll((long long)(lo ? lo : any)) - 1;
      bv = m;
      be = readlane(be, wl);
      if (be == lane) taken |= 1u;
      if (be == lane + WAVE) taken |= 2u;
      sl[r] = bv;
      se[r] = be;
    }
    // weights and ascending-id order (every lane holds the same 8 winners)
    if (lane < K) {
      float den = 0.f;
#pragma unroll
      for (int r = 0; r < K; ++r) den += expf(sl[r] - sl[0]);
      float myl = sl[0];
      int mye = se[0];
#pragma unroll
      for (int r = 1; r < K; ++r)
        if (lane == r) {
          myl = sl[r];
          mye = se[r];
        }
      int rank = 0;
#pragma unroll
      for (int r = 0; r < K; ++r) rank += se[r] < mye;
      sel_e[rank] = mye;
      sel_w[rank] = expf(myl - sl[0]) / den;
    }
  }
  __syncthreads();

  // ---- phase 3: load this workgroup's whole weight share ----
  const int e_j = sel_e[slot];
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
    const float gv = wave_sum(block_dot<FMT>(lds, gbase, xv, xsum));
    const float uv = wave_sum(block_dot<FMT>(lds, gbase + G::PPG * G::GU_ROW, xv, xsum));
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
    gather<2>(p.h + ((part % HREP) * K + slot) * F + tid, F / 2, epoch, p.err, hv2);
    hs[tid] = hv2[0];
    hs[tid + F / 2] = hv2[1];
  }
  __syncthreads();
  {
    const int rl = lane >> 3, sub = lane & 7;       // 8 rows per wavefront, 8 lanes per row
    const int row = wave * 8 + rl;                  // 0..63
    float acc = 0.f;
#pragma unroll
    for (int bi = 0; bi < 3; ++bi) {
      const int b = sub + 8 * bi;                   // 24 blocks per down row
      float hv[QK];
      const float4* hp = (const float4*)(hs + b * QK);
#pragma unroll
      for (int i = 0; i < QK / 4; ++i) {
        const float4 v = hp[i];
        hv[4 * i + 0] = v.x;
        hv[4 * i + 1] = v.y;
        hv[4 * i + 2] = v.z;
        hv[4 * i + 3] = v.w;
      }
      float hsum = 0.f;
#pragma unroll
      for (int i = 0; i < QK; ++i) hsum += hv[i];
      acc += block_dot<FMT>(lds, G::DN_OFF + row * G::DN_ROW + b * G::BB, hv, hsum);
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
    gather<K>(p.y + d, D, epoch, p.err, yv);
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
  a.err = ws.sync + 16;                                   // byte 64
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
