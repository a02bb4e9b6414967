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
// part r = w % 32: 24 gate/up rows and the 64 down rows d = 64r .. 64r+63 of
// the selected expert.  Per layer l:
//  S  every workgroup: gather o_{l-1} (x for l = 0) and z_l = G_l^T o_{l-1};
//     Σ o^2 by a block reduction (every workgroup forms the same inv = 1/rms
//     from the same values in the same order), logits = inv * z_l + bias,
//     top-8 and weights.  o is read and waited for before any weight load
//     leaves the workgroup: queued behind the weight stream, its latency would
//     be that of the whole stream.
//  W  stream the weight share of the selected expert (~153 KB for Q8_0)
//     through registers, the (gate, up) row groups two ahead of
//  H  the gate/up dots (x = in_l = inv * o); publish h_j(f).  Then the down
//     rows and the next layer's gate entries and bias.
//  Y  gather h_j (768 values), the 64 down rows: u_j(d) = w_j y_j(d).
//  O  add u_j(d) (slot 0 also in_l(d)) into the accumulator of o_l(d), and
//     the workgroup's share of z_{l+1} = G_{l+1}^T o_l — sum over its 64 rows
//     of G_{l+1}(d, e) u_j(d) (slot 0: of in_l(d) + u_0(d)) — into the
//     accumulator of z_{l+1}(e).
// Two exchanges sit on each layer's critical path: h (H -> Y), and the
// accumulators (O -> S).
//
// Accumulators.  Every layer of a launch has its own: o_l(d) receives 8
// contributions (one per slot); z_l(e) is kept as 8 partial sums (copy c takes
// the 32 workgroups of slot c; for layer 0, whose z = G_0^T x comes from the 32
// slot-0 workgroups before the first layer, copy c takes the 4 with part % 8 ==
// c), so that no word takes more than 32 adds: hundreds of adds to one word
// queue behind each other for microseconds.  A contribution is a 64-bit
// fetch-add of (rint(v * 2^24) << c) + 1, c = 8 (o) or 12 (z): a fixed-point
// sum with its own count in the low bits, exact and independent of arrival
// order, so the results are bit-reproducible.  An invalid contribution (NaN
// after a wait that gave up, or out of range) adds 2^4 (o) or 2^6 (z) more,
// and a sum with any such part finishes as NaN, so a failure anywhere in a
// launch reaches every later output.  Wavefront 0 adds the o rows and
// wavefronts 1 and 2 the z share, so the two kinds of adds are in flight
// together.  The add that brings the count to its total returns the whole sum:
// that lane decodes it and publishes it (o_l(d) into 8 replicas and into outs,
// a z copy into 8 replicas) as tagged words; the reader sums the 8 z copies
// in copy order.  A contribution to o must stay below 2^27 in magnitude and a
// workgroup's z share below 2^22, so that the sums fit their fields; beyond
// that it counts as invalid and sets bit 1 of the workspace's error word.
// Accumulators start a launch at zero: at its end every workgroup zeroes its
// share of those it used (all of their adds are done once it has passed the
// last layer's S step), except the last layer's o words, which the lane
// completing each one zeroes.
//
// Replicated words: coherent reads of one cache line from hundreds of CUs
// queue behind each other, so published values are copied: o and the z copies
// 8 times (32 pollers per line), h twice (16 pollers per line).  With 1, 2, 4,
// 8, 16 and 32 copies of o and z the layer took 14.58, 14.37, 14.32, 14.31,
// 14.42 and 14.53 us, with 1, 2 and 4 copies of h 14.38, 14.25 and 14.31 us:
// fewer copies mean fewer stores before a value is out, more mean shorter
// poll queues.  Tags are the launch counter + layer + 1.
#include "decode_common.hpp"

namespace moe {
namespace dec {

constexpr int LMAX = 24;        // layers per launch (per-layer pointers ride in the kernel arguments)
constexpr int AREP = 8;         // replicas of o
constexpr int ZREP = 8;         // replicas of the z copies
constexpr int ZC = 8;           // partial copies of z
// Low fields of an accumulator word: a count of contributions (4 bits for o's
// 8, 6 for a z copy's 32) and above it a count of invalid ones; the
// fixed-point sum sits above both.
constexpr int OP = 4, OQ = 8;   // o: count bits, count + invalid-count bits
constexpr int ZP = 6, ZQ = 12;  // z copy
constexpr int ZROWS = DPW / (NT / E);   // rows of one thread's z share (16)
constexpr int ZT0 = WAVE;       // threads ZT0 .. ZT0 + E - 1 add the z share (wavefronts 1, 2)
constexpr float O_LIM = 134217728.0f;   // |contribution| < 2^27: 9 of them * 2^51 < 2^55
constexpr float Z_LIM = 4194304.0f;     // |contribution| < 2^22: 32 of them * 2^46 = 2^51
static_assert(D == 4 * NT, "four o words per thread");
static_assert(NT % E == 0 && DPW % (NT / E) == 0, "z shares");
static_assert(ZC == K && PARTS % ZC == 0, "z copies: one per slot, or part % 8 for layer 0");
static_assert(K < (1 << OP) && K < (1 << (OQ - OP)) && PARTS < (1 << ZP) &&
              PARTS < (1 << (ZQ - ZP)), "count fields");
static_assert(DPW <= WAVE && ZT0 + E <= NT, "o adds on wavefront 0, z adds on the next two");

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
  int32_t* offsets;      // [E+1] or null: the grouping of the last layer's token (one layer)
  int32_t* rows;         // [K] or null
  uint64_t* xa;          // [AREP][D] o replicas
  uint64_t* xz;          // [ZREP][ZC][E] replicas of the z copies
  uint64_t* xc;          // [HREP][K][F] h
  uint64_t* oacc;        // [LMAX][D] o accumulators (zero at launch start)
  uint64_t* zacc;        // [LMAX][ZC][E] z accumulators (zero at launch start)
  uint32_t* epochs;      // [NWG] launch counters
  uint32_t* err;         // bit 0: a poll timed out; bit 1: a value outside the fixed-point range
  int L;
  int prenorm0;
  int residual;          // o_l includes in_l (always in a stack; a single layer may drop it)
  LayerPtrs layer[LMAX];
};

// v * 2^24, rounded, when |v| < lim; otherwise (NaN included) 0, `bad` set and
// the range bit of the error word raised
__device__ inline int64_t fixq(float v, float lim, bool& bad, uint32_t* err) {
  if (!(fabsf(v) < lim)) {
    __hip_atomic_fetch_or(err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bad = true;
    return 0;
  }
  return (int64_t)__builtin_rintf(v * 16777216.0f);
}

// Add a contribution to accumulator *a (count in the low `pbits` bits, invalid
// contributions counted above it, the sum above `qbits`).  Returns true for the
// add that brings the count to `total`, with the finished value (NaN if any
// contribution was invalid).
__device__ inline bool accumulate(uint64_t* a, int64_t q, bool bad, int pbits, int qbits,
                                  uint32_t total, float& out) {
  const uint64_t add = ((uint64_t)q << qbits) + 1u + (bad ? (1ull << pbits) : 0ull);
  const uint64_t old = __hip_atomic_fetch_add(a, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((uint32_t)(old & ((1ull << pbits) - 1u)) != total - 1u) return false;
  const uint64_t sum = old + add;
  const bool invalid = ((sum >> pbits) & ((1ull << (qbits - pbits)) - 1u)) != 0;
  out = invalid ? __builtin_nanf("")
                : (float)((double)((int64_t)sum >> qbits) * (1.0 / 16777216.0));
  return true;
}

template <int FMT>
__global__ __launch_bounds__(NT, 1) void decode_stack_kernel(StackArgs p) {
  using G = Geo<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS_BYTES + 16];  // +16: reads may pass a row end by 2 bytes
  __shared__ float ssred[NWAVE];
  __shared__ __attribute__((aligned(16))) float lg[E];
  __shared__ __align__(16) int top[K];
  __shared__ int sel_e[K];
  __shared__ float sel_w[K];
  __shared__ float s_inv;
  __shared__ float us[DPW];                 // u_j(d) of this workgroup's rows
  __shared__ float vs[DPW];                 // what its z share multiplies
  __shared__ float zred[NT / E][E];

  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int wg = blockIdx.x;
  const int slot = wg / PARTS, part = wg % PARTS;
  const int f0 = part * FPW, dr0 = part * DPW;
  const int ze = tid % E, zq = tid / E;     // z share: expert ze over rows dr0 + 16 zq .. + 15
  uint32_t budget = SPIN_LIMIT;
  const uint32_t base = __hip_atomic_load(p.epochs + wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int L = p.L;

  // Gate entries of the z share and the bias of the coming layer.  Every
  // workgroup loads them (uniform, unconditional loads keep the compiler's wait
  // counts exact).  The bias is kept as loaded (the gate's first values stand in
  // for a missing one) and masked where the logits are formed: using a load
  // right away would make the compiler wait for it, and with it for every weight
  // load before it.
  float gq[ZROWS];
  float b0, b1;
  auto load_gate = [&](const float* Gm, int zq_, int ze_) {
#pragma unroll
    for (int i = 0; i < ZROWS; ++i) gq[i] = Gm[(int64_t)(dr0 + ZROWS * zq_ + i) * E + ze_];
  };
  {
    const LayerPtrs& l0 = p.layer[0];
    load_gate(l0.gate, zq, ze);
    const float* bp = l0.bias ? l0.bias : l0.gate;
    b0 = bp[lane];
    b1 = bp[lane + WAVE];
  }

  // z share: the fp32 values in vs (64 rows) times the gate entries, each
  // thread over 16 rows, then the four row quarters summed in a fixed order;
  // z_partial ends with a barrier, z_add runs on threads ZT0 .. ZT0 + E - 1
  auto z_partial = [&](int zq_, int ze_) {
    float zp = 0.f;
#pragma unroll
    for (int i = 0; i < ZROWS; ++i) zp = fmaf(gq[i], vs[ZROWS * zq_ + i], zp);
    zred[zq_][ze_] = zp;
    __syncthreads();
  };
  auto z_add = [&](int e, int ml, int copy, uint32_t total, uint32_t tag) {
    float z = zred[0][e];
#pragma unroll
    for (int q = 1; q < NT / E; ++q) z += zred[q][e];
    bool bad = false;
    const int64_t q = fixq(z, Z_LIM, bad, p.err);
    float zf = 0.f;
    if (accumulate(p.zacc + ((int64_t)ml * ZC + copy) * E + e, q, bad, ZP, ZQ, total, zf)) {
#pragma unroll 4
      for (int rep = 0; rep < ZREP; ++rep) publish(p.xz + (rep * ZC + copy) * E + e, tag, zf);
    }
  };
  // z_0 = G_0^T x, added by the slot-0 workgroups over their rows
  if (slot == 0) {
    if (tid < DPW) vs[tid] = p.x[dr0 + tid];
    __syncthreads();
    z_partial(zq, ze);
    if (tid >= ZT0 && tid < ZT0 + E) z_add(tid - ZT0, 0, part % ZC, PARTS / ZC, base + 1u);
  }

  for (int l = 0; l < L; ++l) {
    const uint32_t t = base + (uint32_t)l + 1u;
    // per-layer copies of the thread coordinates that the compiler cannot hoist:
    // otherwise it keeps loop-invariant address arithmetic (weight chunk offsets,
    // exchange addresses) live across the whole layer and spills
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid % WAVE, wave = tid / WAVE, ze = tid % E, zq = tid / E;
    const LayerPtrs& lp = p.layer[l];

    // ---- S: o_{l-1} (x before layer 0), z_l, inv, logits, top-8, weights ----
    // Wavefront 0 polls the 8 z copies of its two experts with its share of o
    // (spreading the copies over the wavefronts measured slower).
    const uint64_t* arep = p.xa + (wg % AREP) * D;
    const uint64_t* zrep = p.xz + (wg % ZREP) * ZC * E;
    float xo[4];
    float zv[2] = {0.f, 0.f};
    {
      float pv[2 * ZC + 4];
      if (wave == 0) {
        if (l == 0)
          gather_fn<2 * ZC>([=](int i) { return zrep + (i >> 1) * E + lane + (i & 1) * WAVE; },
                            t, p.err, budget, pv);
        else
          gather_fn<2 * ZC + 4>(
              [=](int i) {
                return i < 2 * ZC ? zrep + (i >> 1) * E + lane + (i & 1) * WAVE
                                  : arep + tid + (i - 2 * ZC) * NT;
              },
              t, p.err, budget, pv);
#pragma unroll
        for (int c = 0; c < ZC; ++c) {             // the copies in copy order
          zv[0] += pv[2 * c];
          zv[1] += pv[2 * c + 1];
        }
      }
      if (l == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xo[i] = p.x[tid + i * NT];
      } else if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xo[i] = pv[2 * ZC + i];
      } else {
        gather_fn<4>([=](int i) { return arep + tid + i * NT; }, t, p.err, budget, xo);
      }
    }
    // o lands in LDS unscaled (inv is known after the barrier); it aliases the
    // gate/up region, which is free until the group stores
    float* xs = (float*)lds;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[tid + i * NT] = xo[i];
      sq = fmaf(xo[i], xo[i], sq);
    }
    sq = wave_sum(sq);
    if (lane == 0) ssred[wave] = sq;
    __syncthreads();
    if (wave == 0) {
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) ss += ssred[w];
      const float inv = (l > 0 || p.prenorm0) ? 1.0f / sqrtf(ss / (float)D + PRENORM_EPS) : 1.0f;
      const float bm = lp.bias ? 1.f : 0.f;
      lg[lane] = fmaf(zv[0], inv, b0 * bm);
      lg[lane + WAVE] = fmaf(zv[1], inv, b1 * bm);
      if (lane < K) top[lane] = -1;
      if (lane == 0) s_inv = inv;
    }
    __syncthreads();
    int win[K];
    top8_slots(lg, top, win);
    const float inv = s_inv;
    // the weight stream needs only this slot's expert; the weights are formed
    // once the stream is on its way
    const int e_j = top8_ascending(win, slot);
    // in_l over this part's rows: slot 0 adds it to o_l
    const float in_row = (slot == 0 && p.residual && tid < DPW) ? xs[dr0 + tid] * inv : 0.f;
    // ---- W + H: stream the weight share two groups ahead of the gate/up dots ----
    // A CU cannot have its whole ~153 KB share in flight: issuing it all at
    // once stalls every wavefront at the issue until most of it has arrived,
    // and the dots would only start after the stream.  So the (gate, up) row
    // groups are issued two ahead of the dots, then the down rows, then the
    // next layer's gate entries and bias.  All loads are unconditional
    // (clamped), which keeps the compiler's wait counts exact.
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
    top8_weights(lg, win, sel_e, sel_w);            // published by the barrier below

    // x = in_l = inv * o as digit planes (all threads, LDS past xs), then this
    // lane's block (block `lane` of the 2048-wide input) into registers
    uint8_t* xdig = lds + D * 4;
    float2* xscl = (float2*)(lds + D * 4 + (D / QK) * 96);
    act_digits_lds<FMT, 4>(xs, inv, D / QK, xdig, xscl);
    __syncthreads();
    const float w_j = sel_w[slot];
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
      // the last layer re-reads its own entries: unconditional loads, see above
      const LayerPtrs& nx = p.layer[min(l + 1, L - 1)];
      load_gate(nx.gate, zq, ze);
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

    // ---- Y: u_j(d) = w_j y_j(d) for 64 down rows ----
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
      if (sub == 0) us[row] = w_j * acc;
    }
    __syncthreads();

    // ---- O: o_l and z_{l+1} accumulators ----
    if (l + 1 < L) {
      if (tid < DPW) vs[tid] = slot == 0 ? in_row + us[tid] : us[tid];
      __syncthreads();
      z_partial(zq, ze);
    }
    if (tid < DPW) {
      const int d = dr0 + tid;
      bool bad = false;
      int64_t q = fixq(us[tid], O_LIM, bad, p.err);
      if (slot == 0) q += fixq(in_row, O_LIM, bad, p.err);
      float o;
      uint64_t* acc = p.oacc + (int64_t)l * D + d;
      if (accumulate(acc, q, bad, OP, OQ, K, o)) {
        p.outs[(int64_t)l * D + d] = o;
        if (l + 1 < L) {
#pragma unroll 4
          for (int rep = 0; rep < AREP; ++rep) publish(p.xa + rep * D + d, t + 1u, o);
        } else {
          // the last layer's word: no other add follows, zero it for the next launch
          __hip_atomic_store(acc, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    } else if (l + 1 < L && tid >= ZT0 && tid < ZT0 + E) {
      z_add(tid - ZT0, l + 1, slot, PARTS, t + 1u);
    }
    // the routing record goes out last: a store waits for its completion at the
    // next wait for a load, and here that is the next exchange
    if (wg == 0 && tid < K) {
      if (p.ids) p.ids[l * K + tid] = sel_e[tid];
      if (p.w) p.w[l * K + tid] = sel_w[tid];
    }
    if (wg == 0 && l + 1 == L) {
      // the grouping of one token: ids ascend, so slot j is flat row j
      if (p.rows && tid < K) p.rows[tid] = tid;
      if (p.offsets && tid <= E) {
        int c = 0;
#pragma unroll
        for (int j = 0; j < K; ++j) c += sel_e[j] < tid;
        p.offsets[tid] = c;
      }
    }
    // every wavefront leaves the layer together: measured faster than letting
    // the early ones start polling while the others still publish
    __syncthreads();
  }

  // Zero this workgroup's share of the accumulators the launch used: every add
  // to o_0 .. o_{L-2} and z_0 .. z_{L-1} is done (this workgroup has read all of
  // them), and the o_{L-1} words were zeroed by the lanes that completed them.
  {
    const int no = (L - 1) * D, nz = L * ZC * E;
    for (int i = wg * NT + tid; i < no + nz; i += NWG * NT) {
      uint64_t* a = i < no ? p.oacc + i : p.zacc + (i - no);
      __hip_atomic_store(a, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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

bool decode_stack_layer_ok(const ExpertsDev& W, int k) {
  if (k != dec::K || W.D != dec::D || W.F != dec::F || W.E != dec::E) return false;
  if (W.fmt != MOE_FMT_Q8_0 && W.fmt != MOE_FMT_Q4) return false;
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  // weight rows are read as 16-byte pieces
  if (!a16(W.gate) || !a16(W.up) || !a16(W.down) || (W.gate_stride & 15) ||
      (W.up_stride & 15) || (W.down_stride & 15))
    return false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  return W.fmt == MOE_FMT_Q8_0 ? dec::stack_fits<MOE_FMT_Q8_0>(dev) : dec::stack_fits<MOE_FMT_Q4>(dev);
}

bool decode_stack_io_ok(const float* x, const float* out) {
  return ((uintptr_t)x & 15) == 0 && ((uintptr_t)out & 15) == 0;
}

hipError_t launch_decode_stack(const float* x, int L, const StackLayer* layers, int fmt,
                               bool prenorm0, bool residual, float* outs, int32_t* ids, float* w,
                               int32_t* offsets, int32_t* rows, const Workspace& ws,
                               hipStream_t s) {
  if (L <= 0 || L > dec::LMAX) return hipErrorInvalidValue;
  dec::StackArgs a{};
  a.x = x;
  a.outs = outs;
  a.ids = ids;
  a.w = w;
  a.offsets = offsets;
  a.rows = rows;
  a.residual = residual ? 1 : 0;
  char* sync = (char*)ws.sync;
  a.err = ws.sync + ERR_WORD_OFF / sizeof(uint32_t);
  a.epochs = (uint32_t*)(sync + 4096);                    // [256] u32
  a.xz = (uint64_t*)(sync + 65536);                       // [ZREP][8][128] u64 (64 KiB)
  a.xc = (uint64_t*)(sync + 327680);                      // [HREP][8][768] u64 (96 KiB)
  a.xa = (uint64_t*)(sync + 524288);                      // [AREP][2048] u64 (128 KiB)
  static_assert(65536 + dec::ZREP * dec::ZC * dec::E * 8 <= 327680 &&
                327680 + dec::HREP * dec::K * dec::F * 8 <= 524288 &&
                524288 + dec::AREP * dec::D * 8 <= STACK_ACC_OFF, "exchange regions");
  // the accumulators sit where no other kernel writes (the small-batch routing
  // starts at ROUTE_SYNC_OFF)
  a.oacc = (uint64_t*)(sync + STACK_ACC_OFF);                     // [24][2048] u64 (384 KiB)
  a.zacc = (uint64_t*)(sync + STACK_ACC_OFF + 393216);            // [24][8][128] u64 (192 KiB)
  static_assert(524288 + 524288 <= STACK_ACC_OFF &&
                STACK_ACC_OFF + 393216 + 196608 <= ROUTE_SYNC_OFF, "sync region");
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
