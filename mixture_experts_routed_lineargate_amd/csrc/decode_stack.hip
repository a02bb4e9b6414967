// Single-token decode through a stack of MoE layers in ONE launch (Qwen3-MoE
// geometry: d_model 2048, d_ff 768, 128 experts, top-8; evidence page, Model
// card).  Each layer is the routed MoE layer with the residual add, and the
// RMSNorm transition sits between layers:
//   in_0 = x (or rmsnorm(x) when the stack continues an earlier one),
//   o_l = in_l + MoE_l(in_l),   in_{l+1} = o_l / sqrt(mean(o_l^2) + 1e-6).
// The warm path then has no host synchronisation and no launch gap between
// layers (evidence page: fewer warm host synchronisations; technical-overview
// page: warm target path router -> resident expert -> combine).
//
// Work split (decode_common.hpp): workgroup w serves expert slot j = w / 32,
// part r = w % 32 (24 gate/up rows, 64 down rows of the selected expert).  The
// 64 router workgroups (eg, ds) = (w % 8, w / 8) also own the 256-row slice ds
// of the residual stream.  Per layer l:
//  R  router workgroup (eg, ds): gather w_j y_j(d) of layer l-1 for its slice
//     (8 words per row, from the 32 workgroups whose down rows cover it), sum
//     them in slot order onto the residual in_{l-1}(d): that is o_{l-1}(d),
//     bit-identical in the 8 workgroups of the slice.  Publish o_{l-1}(d) for
//     32 rows (the broadcast copy, 32 replicas), the partial logits of 16
//     experts over the slice, and the slice's sum of squares.
//  S  every workgroup: gather the partials and sums of squares, form
//     inv = 1/rms, logits = inv * sum_ds partial + bias, top-8 and weights.
//     The o broadcast is read in the same round as the partials and waited
//     for before any weight load leaves the workgroup: queued behind the
//     weight stream, its latency would be that of the whole stream.
//  W  stream the weight share of the selected expert (~153 KB for Q8_0)
//     through registers, the (gate, up) row groups two ahead of
//  H  the gate/up dots (x = in_l = inv * o); publish h_j(f).  Then the down
//     rows and the next layer's gate rows and bias.
//  Y  gather h_j (768 values), the 64 down rows, publish w_j y_j(d).
// Layer 0 runs the same steps with o_{-1} = x (inv = 1 unless the stack
// continues an earlier one).  After the last layer the router workgroups
// gather y once more and write the last output.  Three exchanges sit on each layer's critical path
// (y -> R, R -> S, H -> Y).
//
// Exchange buffers are reused by every layer.  A buffer is rewritten for layer
// l+1 only after its layer-l readers are done, because every publication of
// layer l+1 depends (through the chain of exchanges) on a value that every
// workgroup published after its own layer-l read of that buffer.
#include "decode_common.hpp"

namespace moe {
namespace dec {

constexpr int LMAX = 24;        // layers per launch (per-layer pointers ride in the kernel arguments)
constexpr int AREP = 32;        // replicas of the o broadcast
constexpr int XB_ROW = E + 8;   // [E partial logits][sum of squares][pad]
constexpr int OSUB = SLICE / REG;   // o rows each router workgroup broadcasts (32)
static_assert(OSUB * AREP == 2 * NT, "two broadcast stores per thread");
static_assert(PREP % REG == 0, "sum-of-squares replicas split evenly");
static_assert(D == 4 * NT, "four broadcast words per thread");

struct LayerPtrs {
  const float* gate;     // [D][E] fp32
  const float* bias;     // [E] fp32 or null
  const uint8_t* wg;
  const uint8_t* wu;
  const uint8_t* wd;
  int64_t sg, su, sd;    // expert strides (bytes)
};

struct StackArgs {
  const float* x;        // [D] layer-0 input (the previous output when prenorm0)
  float* outs;           // [L][D] o_l
  int32_t* ids;          // [L][K] or null
  float* w;              // [L][K] or null
  uint64_t* xb;          // [PREP][RDS][XB_ROW] partial logits + sums of squares
  uint64_t* xa;          // [AREP][D] o broadcast
  uint64_t* xc;          // [HREP][K][F] h
  uint64_t* xd;          // [K][D] w_j y_j
  uint32_t* epochs;      // [NWG] launch counters
  uint32_t* err;         // poll timeout flag
  int L;
  int prenorm0;
  LayerPtrs layer[LMAX];
};

template <int FMT>
__global__ __launch_bounds__(NT, 1) void decode_stack_kernel(StackArgs p) {
  using G = Geo<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES + 16];  // +16: reads may pass a row end by 2 bytes
  __shared__ float red[NT];
  __shared__ float slice_o[SLICE];
  __shared__ float rsum[REPG];
  __shared__ float ssred[NWAVE];
  __shared__ __attribute__((aligned(16))) float lg[E];
  __shared__ __align__(16) int top[K];
  __shared__ int sel_e[K];
  __shared__ float sel_w[K];
  __shared__ float s_inv;

  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int wg = blockIdx.x;
  const int slot = wg / PARTS, part = wg % PARTS;
  const bool router = wg < RW;
  const int eg = wg % REG, ds = (wg % RW) / REG;
  const int el = tid % REPG, rg = tid / REPG;
  const int f0 = part * FPW, dr0 = part * DPW;
  uint32_t budget = SPIN_LIMIT;
  const uint32_t base = __hip_atomic_load(p.epochs + wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int L = p.L;

  // router state: thread t < SLICE owns row d = ds*SLICE + t of the residual stream
  float o_reg = 0.f;    // o_{l-1}(d); x(d) before layer 0
  float in_reg = 0.f;   // in_{l-1}(d)
  if (router && tid < SLICE) o_reg = p.x[ds * SLICE + tid];
  // Gate rows and bias of the current layer.  Every workgroup loads them (the
  // non-router ones re-read a router workgroup's rows and drop them):
  // conditional loads would make later waits drain the weight stream too.
  // The bias is kept as loaded (the gate's first values stand in for a missing
  // one) and masked where the logits are formed: using a load right away would
  // make the compiler wait for it, and with it for every weight load before it.
  float gq[RROWS];
  float b0, b1;
  {
    const LayerPtrs& l0 = p.layer[0];
#pragma unroll
    for (int r = 0; r < RROWS; ++r) gq[r] = l0.gate[(int64_t)(ds * SLICE + rg * RROWS + r) * E + eg * REPG + el];
    const float* bp = l0.bias ? l0.bias : l0.gate;
    b0 = bp[lane];
    b1 = bp[lane + WAVE];
  }

  for (int l = 0; l < L; ++l) {
    const uint32_t t = base + (uint32_t)l + 1u;
    // per-layer copies of the thread coordinates that the compiler cannot hoist:
    // otherwise it keeps loop-invariant address arithmetic (weight chunk offsets,
    // exchange addresses) live across the whole layer and spills
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid % WAVE, wave = tid / WAVE, el = tid % REPG, rg = tid / REPG;
    const LayerPtrs& lp = p.layer[l];

    // ---- R: o_{l-1} of this slice, partial logits, publish ----
    if (router) {
      if (l > 0 && tid < SLICE) {
        const int d = ds * SLICE + tid;
        float yv[K];
        gather<K>(p.xd + d, D, t - 1u, p.err, budget, yv);
        float s = in_reg;
#pragma unroll
        for (int j = 0; j < K; ++j) s += yv[j];
        o_reg = s;
        if (tid / OSUB == eg) p.outs[(int64_t)(l - 1) * D + d] = s;
      }
      float sq = 0.f;
      if (tid < SLICE) {
        slice_o[tid] = o_reg;
        sq = o_reg * o_reg;
      }
      sq = wave_sum(sq);
      if (lane == 0) ssred[wave] = sq;
      __syncthreads();
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < RROWS; ++r) acc = fmaf(slice_o[rg * RROWS + r], gq[r], acc);
      red[tid] = acc;
      // the broadcast copy of o goes out first: consumers read it after the partials
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = tid + i * NT;
        const int rep = q / OSUB, dd = q % OSUB;
        publish(p.xa + rep * D + ds * SLICE + eg * OSUB + dd, t, slice_o[eg * OSUB + dd]);
      }
      __syncthreads();
      if (wave == 0) {
        // red[g*16 + e]: lane l sums row groups l/16, l/16 + 4, ... for expert l%16,
        // then the four lane quarters are added
        float sum = 0.f;
#pragma unroll
        for (int g = 0; g < RGRP / 4; ++g) sum += red[(4 * g + (lane >> 4)) * REPG + (lane & 15)];
        sum += __shfl_xor(sum, 32);
        sum += __shfl_xor(sum, 16);
        if (lane < REPG) rsum[lane] = sum;
      }
      __syncthreads();
      {
        const int rep = tid / REPG;
        publish(p.xb + (rep * RDS + ds) * XB_ROW + eg * REPG + el, t, rsum[el]);
      }
      if (tid < PREP / REG) {
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) ss += ssred[w];
        const int rep = eg + REG * tid;
        publish(p.xb + (rep * RDS + ds) * XB_ROW + E, t, ss);
      }
    }

    // ---- S: logits, top-8, weights ----
    // Every thread polls its share of the o broadcast (wavefront 0 together with
    // the partials and sums of squares).  The o reads complete before any weight
    // load leaves the workgroup: queued behind the weight stream, their latency
    // would be that of the whole stream.
    const uint64_t* xbrep = p.xb + (wg % PREP) * RDS * XB_ROW;
    const uint64_t* arep = p.xa + (wg % AREP) * D;
    float xo[4];
    if (wave == 0) {
      // partials [ds][e] (e = lane, lane + 64), the sum of squares of slice lane % 8,
      // and this thread's four o words, in one poll loop
      float pv[2 * RDS + 1 + 4];
      gather_fn<2 * RDS + 1 + 4>(
          [=](int i) {
            return i < 2 * RDS ? xbrep + (i >> 1) * XB_ROW + lane + (i & 1) * WAVE
                 : i == 2 * RDS ? xbrep + (lane % RDS) * XB_ROW + E
                                : arep + tid + (i - 2 * RDS - 1) * NT;
          },
          t, p.err, budget, pv);
#pragma unroll
      for (int i = 0; i < 4; ++i) xo[i] = pv[2 * RDS + 1 + i];
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < RDS; ++s) ss += readlane(pv[2 * RDS], s);
      const float inv = (l > 0 || p.prenorm0) ? 1.0f / sqrtf(ss / (float)D + PRENORM_EPS) : 1.0f;
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int s = 0; s < RDS; ++s) {
        v0 += pv[2 * s];
        v1 += pv[2 * s + 1];
      }
      const float bm = lp.bias ? 1.f : 0.f;
      lg[lane] = fmaf(v0, inv, b0 * bm);
      lg[lane + WAVE] = fmaf(v1, inv, b1 * bm);
      if (lane < K) top[lane] = -1;
      if (lane == 0) s_inv = inv;
    } else {
      gather_fn<4>([=](int i) { return arep + tid + i * NT; }, t, p.err, budget, xo);
    }
    // o lands in LDS unscaled (inv is known after the barrier); it aliases the
    // gate/up region, which is free until the group stores
    float* xs = (float*)lds;
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[tid + i * NT] = xo[i];
    __syncthreads();
    select_top8_block(lg, top, sel_e, sel_w);
    const float inv = s_inv;
    const int e_j = min(max(sel_e[slot], 0), E - 1);
    const float w_j = sel_w[slot];
    if (router && tid < SLICE) in_reg = o_reg * inv;

    // ---- W + H: stream the weight share two groups ahead of the gate/up dots ----
    // A CU cannot have its whole ~153 KB share in flight: issuing it all at
    // once stalls every wavefront at the issue until most of it has arrived,
    // and the dots would only start after the stream.  So the (gate, up) row
    // groups are issued two ahead of the dots, then the down rows, then the
    // next layer's gate rows and bias.  All loads are unconditional (clamped),
    // which keeps the compiler's wait counts exact.
    const uint8_t* gsrc = lp.wg + (int64_t)e_j * lp.sg + (int64_t)f0 * G::GU_ROW;
    const uint8_t* usrc = lp.wu + (int64_t)e_j * lp.su + (int64_t)f0 * G::GU_ROW;
    const uint8_t* dsrc = lp.wd + (int64_t)e_j * lp.sd + (int64_t)dr0 * G::DN_ROW;
    auto load_group = [&](int g, u32x4* dst) {
#pragma unroll
      for (int it = 0; it < G::GRP_ITERS; ++it) {
        const int c = min(it * NT + tid, G::GRP_CHUNKS - 1);
        constexpr int half = G::GRP_CHUNKS / 2;       // gate rows first, then up rows
        const int64_t row_off = (int64_t)(g * G::PPG) * G::GU_ROW;
        const uint8_t* src = c < half ? gsrc + row_off + 16 * c : usrc + row_off + 16 * (c - half);
        dst[it] = __builtin_nontemporal_load((const u32x4*)src);
      }
    };
    u32x4 ga[G::GRP_ITERS], gb[G::GRP_ITERS];
    u32x4 dn[G::DN_ITERS];
    load_group(0, ga);
    load_group(1, gb);

    // x = in_l = inv * o as digit planes (all threads, LDS past xs), then this
    // lane's block (block `lane` of the 2048-wide input) into registers
    uint8_t* xdig = lds + D * 4;
    float2* xscl = (float2*)(lds + D * 4 + (D / QK) * 96);
    act_digits_lds<FMT, 4>(xs, inv, D / QK, xdig, xscl);
    __syncthreads();
    ActDig xd;
    load_dig(xdig, xscl, lane, xd);
    __syncthreads();                                  // xs consumed

    // group g: rows to LDS, then wavefront w computes the (gate, up) pair w
    auto gate_up = [&](int g, const u32x4* src) {
#pragma unroll
      for (int it = 0; it < G::GRP_ITERS; ++it) {
        const int c = it * NT + tid;
        if (c < G::GRP_CHUNKS) *(u32x4*)(lds + g * G::GRP_BYTES + 16 * c) = src[it];
      }
      __syncthreads();
      const uint32_t gbase = g * G::GRP_BYTES + wave * G::GU_ROW + lane * G::BB;
      const float gv = wave_sum(block_dot_dig<FMT>(lds, gbase, xd));
      const float uv = wave_sum(block_dot_dig<FMT>(lds, gbase + G::PPG * G::GU_ROW, xd));
      if (lane < HREP)
        publish(p.xc + (lane * K + slot) * F + f0 + g * G::PPG + wave, t, silu(gv) * uv);
    };
    static_assert(G::NGRP == 3, "the pipeline below is written for three groups");
    gate_up(0, ga);
    load_group(2, ga);
    gate_up(1, gb);
#pragma unroll
    for (int it = 0; it < G::DN_ITERS; ++it) {
      const int c = min(it * NT + tid, G::DN_CHUNKS - 1);
      dn[it] = __builtin_nontemporal_load((const u32x4*)(dsrc + 16 * c));
    }
    {
      // the last layer re-reads its own rows: unconditional loads, see above
      const LayerPtrs& nx = p.layer[min(l + 1, L - 1)];
#pragma unroll
      for (int r = 0; r < RROWS; ++r)
        gq[r] = nx.gate[(int64_t)(ds * SLICE + rg * RROWS + r) * E + eg * REPG + el];
      const float* bp = nx.bias ? nx.bias : nx.gate;
      b0 = bp[lane];
      b1 = bp[lane + WAVE];
    }
    gate_up(2, ga);
#pragma unroll
    for (int it = 0; it < G::DN_ITERS; ++it) {
      const int c = it * NT + tid;
      if (c < G::DN_CHUNKS) *(u32x4*)(lds + G::DN_OFF + 16 * c) = dn[it];
    }

    // ---- Y: w_j y_j(d) for 64 down rows ----
    __syncthreads();                                  // every wave is done with the gate/up region
    float* hs = (float*)lds;                          // h_j [F], reuses the gate/up region
    if (tid < F / 2) {
      float hv2[2];
      gather<2>(p.xc + ((part % HREP) * K + slot) * F + tid, F / 2, t, p.err, budget, hv2);
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
      if (sub == 0) publish(p.xd + slot * D + dr0 + row, t, w_j * acc);
    }
    // the routing record goes out last: a store waits for its completion at the
    // next wait for a load, and here that is the next exchange
    if (wg == 0 && tid < K) {
      if (p.ids) p.ids[l * K + tid] = sel_e[tid];
      if (p.w) p.w[l * K + tid] = sel_w[tid];
    }
  }

  // ---- the last layer's output ----
  if (router && tid < SLICE) {
    const int d = ds * SLICE + tid;
    float yv[K];
    gather<K>(p.xd + d, D, base + (uint32_t)L, p.err, budget, yv);
    float s = in_reg;
#pragma unroll
    for (int j = 0; j < K; ++j) s += yv[j];
    if (tid / OSUB == eg) p.outs[(int64_t)(L - 1) * D + d] = s;
  }
  if (tid == 0)
    __hip_atomic_store(p.epochs + wg, base + (uint32_t)L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT>
static bool stack_fits(int dev) {
  static int cache[64][2];
  if (dev < 0 || dev >= 64) return false;
  int& c = cache[dev][FMT];
  if (c == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_stack_kernel<FMT>, NT, 0) !=
            hipSuccess) {
      c = -1;
    } else {
      c = (cus * per >= NWG) ? 1 : -1;
    }
  }
  return c == 1;
}

}  // namespace dec

int decode_stack_max_layers() { return dec::LMAX; }

bool decode_stack_supported(int fmt) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  return fmt == MOE_FMT_Q8_0 ? dec::stack_fits<MOE_FMT_Q8_0>(dev) : dec::stack_fits<MOE_FMT_Q4>(dev);
}

hipError_t launch_decode_stack(const float* x, int L, const StackLayer* layers, int fmt,
                               bool prenorm0, float* outs, int32_t* ids, float* w,
                               const Workspace& ws, hipStream_t s) {
  if (L <= 0 || L > dec::LMAX) return hipErrorInvalidValue;
  dec::StackArgs a{};
  a.x = x;
  a.outs = outs;
  a.ids = ids;
  a.w = w;
  char* sync = (char*)ws.sync;
  a.err = ws.sync + ERR_WORD_OFF / sizeof(uint32_t);
  a.epochs = (uint32_t*)(sync + 4096);                    // [256] u32, shared with the layer kernel
  a.xb = (uint64_t*)(sync + 65536);                       // [32][8][136] u64 (272 KiB)
  a.xc = (uint64_t*)(sync + 65536 + 278528);              // [4][8][768] u64 (192 KiB)
  a.xd = (uint64_t*)(sync + 65536 + 278528 + 196608);     // [8][2048] u64 (128 KiB)
  a.xa = (uint64_t*)(sync + 65536 + 278528 + 196608 + 131072);  // [32][2048] u64 (512 KiB)
  static_assert(65536 + 278528 + 196608 + 131072 + 524288 <= SYNC_BYTES, "sync region");
  static_assert(dec::PREP * dec::RDS * dec::XB_ROW * 8 == 278528, "xb size");
  a.L = L;
  a.prenorm0 = prenorm0 ? 1 : 0;
  for (int l = 0; l < L; ++l) {
    const StackLayer& sl = layers[l];
    a.layer[l] = dec::LayerPtrs{sl.gate, sl.bias, sl.W.gate, sl.W.up, sl.W.down,
                                sl.W.gate_stride, sl.W.up_stride, sl.W.down_stride};
  }
  if (fmt == MOE_FMT_Q8_0)
    hipLaunchKernelGGL(dec::decode_stack_kernel<MOE_FMT_Q8_0>, dim3(dec::NWG), dim3(dec::NT), 0, s, a);
  else
    hipLaunchKernelGGL(dec::decode_stack_kernel<MOE_FMT_Q4>, dim3(dec::NWG), dim3(dec::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
