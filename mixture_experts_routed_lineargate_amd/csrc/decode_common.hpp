// Pieces of the single-token decode kernel (one or more layers per launch) for
// the Qwen3-MoE geometry: d_model 2048, d_ff 768, 128 experts, top-8 (evidence
// page, Model card); the exchange and block-dot helpers also serve the
// attention-side primitives.
//
// The decode kernel runs 256 workgroups of 512 threads, one per CU, all
// resident at once.  Workgroup w serves expert slot j = w / 32 and part
// r = w % 32 of that expert: gate/up rows f = 24r..24r+23 and down rows
// d = 64r..64r+63.
//
// Exchange between workgroups: every published value is a 64-bit word
// (tag << 32 | fp32 bits) written with an agent-scope store and read with
// agent-scope loads, which on gfx950 are coherent across the XCDs' L2 caches,
// so consumers poll the data itself and need no grid barrier.  Tags come from
// a per-workgroup launch counter kept in the workspace (all workgroups run
// every launch, so their counters agree; the workspace starts zeroed).  Every
// poll loop draws on a per-thread budget for the whole launch: once it is
// spent, an error flag is raised and later waits return at once, so a launch
// always ends.
//
// Dequant in registers: lane b of a wavefront owns block b of a 2048-wide row
// (64 blocks = 64 lanes).  The 34-byte (Q8_0) or 18-byte (Q4) block is read as
// 4-byte-aligned dwords from LDS and realigned with v_alignbyte; int8 codes are
// biased to unsigned (xor 0x80) so one v_cvt_f32_ubyte converts a byte, and
// the bias is removed with the block's activation sum:
//   sum_i q_i x_i = sum_i (q_i + 128) x_i - 128 sum_i x_i   (Q8_0)
//   sum_i (q_i - 8) x_i = sum_i q_i x_i - 8 sum_i x_i        (Q4)
// then multiplied by the fp16 block scale.  Accumulation is fp32.
#pragma once

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
constexpr int HREP = 2;              // replicas of h
static_assert(FPW * PARTS == F && DPW * PARTS == D, "split");
static_assert(D / QK == WAVE, "one block per lane for gate/up rows");
static_assert(E == 2 * WAVE, "two logits per lane");

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
  static_assert(LDS_BYTES + 16 + 6144 <= 160 * 1024, "LDS budget");
  static_assert(D * 4 <= 2 * GU_BYTES, "the input row fits in the gate/up region");
  static_assert(F * 4 <= 2 * GU_BYTES, "h staging fits in the gate/up region");
};

constexpr uint32_t SPIN_LIMIT = 1u << 20;   // poll rounds per thread per launch

__device__ inline uint64_t tag(uint32_t t, float v) {
  return ((uint64_t)t << 32) | (uint64_t)__float_as_uint(v);
}

__device__ inline void publish(uint64_t* p, uint32_t t, float v) {
  __hip_atomic_store(p, tag(t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t peek(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Re-read words I..N-1 of a wait (expanded at compile time, so the words stay
// in registers whatever N is).  Every word is re-read, ready or not: a
// conditional re-read would make the compiler wait for each load before the
// next one is issued, one memory latency per straggler.
template <int I, int N, typename AddrFn>
__device__ inline void repoll(uint64_t* v, AddrFn addr) {
  if constexpr (I < N) {
    v[I] = peek(addr(I));
    repoll<I + 1, N>(v, addr);
  }
}

// Finish a wait on N tagged words whose first reads are already in v: poll
// (word i lives at addr(i)) until all carry tag t, then return the values.
// Spends at most `budget` rounds (shared by every wait of the launch).  A wait
// that runs out of budget sets the error word and returns NaN for every word,
// so whatever it feeds (logits, weights, h, outputs) is NaN, never stale data;
// the selections clamp their ids into [0, E), so addressing stays in bounds.
template <int N, typename AddrFn>
__device__ inline void gather_finish(uint64_t* v, AddrFn addr, uint32_t t, uint32_t* err,
                                     uint32_t& budget, float* out) {
  bool timed_out = false;
  for (;;) {
    bool ready = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ready &= (uint32_t)(v[i] >> 32) == t;
    if (ready) break;
    if (budget == 0) {
      __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // keeps bit 1
      timed_out = true;
      break;
    }
    --budget;
    __builtin_amdgcn_s_sleep(4);
    repoll<0, N>(v, addr);
  }
#pragma unroll
  for (int i = 0; i < N; ++i)
    out[i] = timed_out ? __builtin_nanf("") : __uint_as_float((uint32_t)v[i]);
}

// Wait until the N tagged words at addr(i) all carry tag t; all N loads of a
// round are in flight together.
template <int N, typename AddrFn>
__device__ inline void gather_fn(AddrFn addr, uint32_t t, uint32_t* err, uint32_t& budget,
                                 float* out) {
  uint64_t v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = peek(addr(i));
  gather_finish<N>(v, addr, t, err, budget, out);
}

template <int N>
__device__ inline void gather(const uint64_t* base, int stride, uint32_t t, uint32_t* err,
                              uint32_t& budget, float* out) {
  gather_fn<N>([=](int i) { return base + i * stride; }, t, err, budget, out);
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

// ---------------------------------------------------------------------------
// Integer dot products on v_dot4_i32_i8.  An activation block (32 values) is
// held as fixed point relative to its largest magnitude: with 2^k > max|v|,
// X_i = rint(v_i * 2^(22-k)) (|X_i| <= 2^22, error <= 2^-22 * max|v| per value)
// and v_i ~= s * X_i, s = 2^(k-22).  X_i is split into three signed 8-bit digits,
// X_i = 65536 a_i + 256 b_i + c_i, so sum_i q_i X_i is three exact int32 dot
// products of the raw int8 codes (Q8_0) or nibbles (Q4) with the digit planes;
// one fp32 combination and the two scales finish the block.  Digit dword j
// holds the elements that weight dword j meets: Q8_0 elements 4j..4j+3;
// Q4 even dwords 2i hold elements 8i, 8i+2, 8i+4, 8i+6 (the low nibbles of
// weight dword i), odd dwords 2i+1 the elements 8i+1, 8i+3, ... (high nibbles).
// ---------------------------------------------------------------------------
struct ActDig {
  uint32_t a[8], b[8], c[8];  // digit planes
  float s;                    // block scale 2^(k-22)
  int32_t sx;                 // sum_i X_i (the Q4 offset term)
};

// element held by byte n of digit dword j
template <int FMT>
__host__ __device__ constexpr int dig_elem(int j, int n) {
  return FMT == MOE_FMT_Q8_0 ? 4 * j + n : 8 * (j >> 1) + 2 * n + (j & 1);
}

__device__ inline int32_t sext8(int32_t v) { return ((v & 0xff) ^ 0x80) - 0x80; }

// fixed-point exponent shift for a block whose largest magnitude is m
__device__ inline int dig_shift(float m) { return 22 - __builtin_amdgcn_frexp_expf(m); }

// digits (a, b, c) of X, |X| <= 2^22
__device__ inline void split3(int32_t X, int32_t& a, int32_t& b, int32_t& c) {
  c = sext8(X);
  const int32_t X1 = (X - c) >> 8;
  b = sext8(X1);
  a = (X1 - b) >> 8;
}

// One lane turns its 32 activations into digit planes.
template <int FMT>
__device__ inline void act_digits(const float* v, ActDig& d) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < QK; ++i) m = fmaxf(m, fabsf(v[i]));
  const int sh = dig_shift(m);
  d.s = __builtin_amdgcn_ldexpf(1.0f, -sh);
  int32_t sx = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t pa = 0, pb = 0, pc = 0;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int32_t X = (int32_t)__builtin_rintf(__builtin_amdgcn_ldexpf(v[dig_elem<FMT>(j, n)], sh));
      sx += X;
      int32_t a, b, c;
      split3(X, a, b, c);
      pa |= (uint32_t)(a & 0xff) << (8 * n);
      pb |= (uint32_t)(b & 0xff) << (8 * n);
      pc |= (uint32_t)(c & 0xff) << (8 * n);
    }
    d.a[j] = pa;
    d.b[j] = pb;
    d.c[j] = pc;
  }
  d.sx = sx;
}

// sum_i w_i v_i for one LDS-resident weight block against a digit block.
template <int FMT>
__device__ inline float block_dot_dig(const uint8_t* lds, uint32_t blk_off, const ActDig& d) {
  const uint32_t odd = (blk_off >> 1) & 1u;          // block start is 2 mod 4
  const uint32_t a4 = blk_off - 2u * odd;             // 4-aligned
  int32_t sa = 0, sb = 0, sc = 0;
  uint32_t sbits;
  if constexpr (FMT == MOE_FMT_Q8_0) {
    uint32_t dw[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) dw[i] = lds_u32(lds, a4 + 4u * i);
    sbits = odd ? (dw[0] >> 16) : (dw[0] & 0xffffu);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t q = odd ? dw[i + 1] : __builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2);
      sa = __builtin_amdgcn_sdot4((int)q, (int)d.a[i], sa, false);
      sb = __builtin_amdgcn_sdot4((int)q, (int)d.b[i], sb, false);
      sc = __builtin_amdgcn_sdot4((int)q, (int)d.c[i], sc, false);
    }
  } else {
    uint32_t dw[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) dw[i] = lds_u32(lds, a4 + 4u * i);
    sbits = odd ? (dw[0] >> 16) : (dw[0] & 0xffffu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t n = odd ? dw[i + 1] : __builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2);
      const uint32_t lo = n & 0x0f0f0f0fu, hi = (n >> 4) & 0x0f0f0f0fu;   // codes 0..15
      sa = __builtin_amdgcn_sdot4((int)lo, (int)d.a[2 * i], sa, false);
      sa = __builtin_amdgcn_sdot4((int)hi, (int)d.a[2 * i + 1], sa, false);
      sb = __builtin_amdgcn_sdot4((int)lo, (int)d.b[2 * i], sb, false);
      sb = __builtin_amdgcn_sdot4((int)hi, (int)d.b[2 * i + 1], sb, false);
      sc = __builtin_amdgcn_sdot4((int)lo, (int)d.c[2 * i], sc, false);
      sc = __builtin_amdgcn_sdot4((int)hi, (int)d.c[2 * i + 1], sc, false);
    }
    sc -= 8 * d.sx;                                   // value = d * (q - 8)
  }
  const float r = fmaf((float)sa, 65536.0f, fmaf((float)sb, 256.0f, (float)sc));
  return half_bits_to_float((uint16_t)sbits) * d.s * r;
}

// Digit planes from registers: piece t (elements EPT*t .. EPT*t + EPT-1, block
// t*EPT/32) is held by a lane whose wavefront holds the block's other pieces on
// the adjacent lanes (reduced with DPP); `on` is false for pieces past the
// last block.  Writes dig[blk][3 planes][8 dwords] (bytes) and scl[blk] =
// (s, sx) to LDS; the caller places a barrier after.  Every lane of the
// wavefront must call it.
template <int FMT, int EPT>
__device__ inline void act_digits_reg(const float* x, bool on, int t, uint8_t* dig, float2* scl) {
  static_assert(EPT == 2 || EPT == 4, "8 or 16 threads per block");
  constexpr int TPB = QK / EPT;
  const int blk = t / TPB, e0 = EPT * (t % TPB);
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmaxf(m, fabsf(x[i]));
  m = fmaxf(m, dpp<DPP_QUAD_1032>(m));
  m = fmaxf(m, dpp<DPP_QUAD_2301>(m));
  m = fmaxf(m, dpp<DPP_ROW_HALF_MIRROR>(m));
  if constexpr (TPB == 16) m = fmaxf(m, dpp<DPP_ROW_MIRROR>(m));
  const int sh = dig_shift(m);
  int32_t X[EPT];
  int32_t sx = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    X[i] = (int32_t)__builtin_rintf(__builtin_amdgcn_ldexpf(x[i], sh));
    sx += X[i];
  }
  sx += dpp<DPP_QUAD_1032>(sx);
  sx += dpp<DPP_QUAD_2301>(sx);
  sx += dpp<DPP_ROW_HALF_MIRROR>(sx);
  if constexpr (TPB == 16) sx += dpp<DPP_ROW_MIRROR>(sx);
  if (!on) return;
  uint8_t* base = dig + blk * 96;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = e0 + i;
    // position of element e: digit dword j, byte n (inverse of dig_elem)
    const int j = FMT == MOE_FMT_Q8_0 ? e >> 2 : 2 * (e >> 3) + (e & 1);
    const int n = FMT == MOE_FMT_Q8_0 ? e & 3 : (e & 7) >> 1;
    int32_t a, b, c;
    split3(X[i], a, b, c);
    base[0 * 32 + 4 * j + n] = (uint8_t)a;
    base[1 * 32 + 4 * j + n] = (uint8_t)b;
    base[2 * 32 + 4 * j + n] = (uint8_t)c;
  }
  if (t % TPB == 0) scl[blk] = make_float2(__builtin_amdgcn_ldexpf(1.0f, -sh), __int_as_float(sx));
}

// Digit planes of nblk activation blocks of v*scale, built cooperatively from
// LDS: thread t of the first nblk*32/EPT threads takes EPT consecutive elements
// (act_digits_reg's piece t).  Every thread of the workgroup must call it.
template <int FMT, int EPT>
__device__ inline void act_digits_lds(const float* v, float scale, int nblk, uint8_t* dig,
                                      float2* scl) {
  constexpr int TPB = QK / EPT;
  const int t = threadIdx.x;
  const bool on = t < TPB * nblk;
  float x[EPT];
  if constexpr (EPT == 4) {
    const float4 q = on ? *(const float4*)(v + 4 * t) : make_float4(0.f, 0.f, 0.f, 0.f);
    x[0] = q.x * scale; x[1] = q.y * scale; x[2] = q.z * scale; x[3] = q.w * scale;
  } else {
    const float2 q = on ? *(const float2*)(v + 2 * t) : make_float2(0.f, 0.f);
    x[0] = q.x * scale; x[1] = q.y * scale;
  }
  act_digits_reg<FMT, EPT>(x, on, t, dig, scl);
}

// Load block blk of act_digits_lds's output.
__device__ inline void load_dig(const uint8_t* dig, const float2* scl, int blk, ActDig& d) {
  const u32x4* p = (const u32x4*)(dig + blk * 96);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 va = p[i], vb = p[2 + i], vc = p[4 + i];
    d.a[4 * i + 0] = va.x; d.a[4 * i + 1] = va.y; d.a[4 * i + 2] = va.z; d.a[4 * i + 3] = va.w;
    d.b[4 * i + 0] = vb.x; d.b[4 * i + 1] = vb.y; d.b[4 * i + 2] = vb.z; d.b[4 * i + 3] = vb.w;
    d.c[4 * i + 0] = vc.x; d.c[4 * i + 1] = vc.y; d.c[4 * i + 2] = vc.z; d.c[4 * i + 3] = vc.w;
  }
  const float2 sc = scl[blk];
  d.s = sc.x;
  d.sx = __float_as_int(sc.y);
}

// Top-8 of E = 128 logits by rank counting, spread over the whole workgroup
// (k rounds of a wave arg-max on one wavefront cost about 1.5 us per layer).
// Another logit outranks e if it is larger, or equal with a lower index (the
// router's tie-break), so the ranks are a strict total order and expert e is
// selected iff rank(e) < K.  The caller has written lg[E] to LDS (16-byte
// aligned) and set top[j] = -1 for j < K (top 16-byte aligned), followed by a
// barrier.  Thread t (all NT = 4E threads) compares logit e = t / 4 with logits
// 32*(t%4) .. +31.  The first pass counts only the logits >= lg[e]; less one
// (e itself) that is rank(e) whenever no other logit equals lg[e].  A group of m >= 2 equal logits below c
// larger ones all land on slot c + m - 1 and leave slot c empty, so when all K
// slots are filled no tie reaches the top K and the slots hold the exact ranks
// (a NaN logit counts nothing and takes no slot).  Otherwise a second pass ranks
// with the full comparison; every slot is then preset to its own index,
// so the selected ids are in [0, E) whatever the logits hold.  Returns after a
// barrier with the slots final, as 8 wavefront-uniform ids in rank order.
__device__ inline void top8_slots(const float* lg, int* top, int (&t)[K]) {
  static_assert(NT == 4 * E, "four threads per logit");
  static_assert(K == 8, "the slots are read as two int4");
  const int tid = threadIdx.x;
  const int e = tid >> 2, q = tid & 3;
  const float le = lg[e];
  {
    // every LDS read is issued before the first compare, so the reads overlap
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *(const float4*)(lg + 32 * q + 4 * i);
    int ge = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) ge += (v[i].x >= le) + (v[i].y >= le) + (v[i].z >= le) + (v[i].w >= le);
    ge += dpp<DPP_QUAD_1032>(ge);
    ge += dpp<DPP_QUAD_2301>(ge);
    if (q == 0 && ge >= 1 && ge <= K) top[ge - 1] = e;
  }
  __syncthreads();
  int4 ta = *(const int4*)top, tb = *(const int4*)(top + 4);
  if (min(min(min(ta.x, ta.y), min(ta.z, ta.w)), min(min(tb.x, tb.y), min(tb.z, tb.w))) < 0) {
    // a slot is empty: exact ranks, with the index tie-break
    __syncthreads();                                   // every thread has read the slots
    if (tid < K) top[tid] = tid;
    __syncthreads();
    int cnt = 0;
#pragma unroll 1
    for (int i = 0; i < 32; ++i) {
      const int o = 32 * q + i;
      const float lo = lg[o];
      cnt += (lo > le) | ((lo == le) & (o < e));
    }
    cnt += dpp<DPP_QUAD_1032>(cnt);
    cnt += dpp<DPP_QUAD_2301>(cnt);
    if (q == 0 && cnt < K) top[cnt] = e;
    __syncthreads();
    ta = *(const int4*)top;
    tb = *(const int4*)(top + 4);
  }
  const int v[K] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
#pragma unroll
  for (int r = 0; r < K; ++r) t[r] = __builtin_amdgcn_readfirstlane(min(max(v[r], 0), E - 1));
}

// The id of slot j of the winners in ascending id order (t in rank order, as
// top8_slots returns it): lane r < K ranks winner r among the 8, one ballot
// finds the lane whose rank is j (the ids are distinct).
__device__ inline int top8_ascending(const int (&t)[K], int j) {
  const int lane = threadIdx.x % WAVE;
  int tl = t[0];
#pragma unroll
  for (int r = 1; r < K; ++r) tl = (lane & (K - 1)) == r ? t[r] : tl;
  int c = 0;
#pragma unroll
  for (int q = 0; q < K; ++q) c += t[q] < tl;
  const uint64_t m = __ballot(lane < K && min(c, K - 1) == j);
  return m ? __builtin_amdgcn_readlane(tl, __builtin_ctzll(m)) : t[j];
}

// Wavefront 0: sel_e / sel_w = the winners in ascending id and their
// renormalised softmax weights (lane j < K takes winner j in rank order; the
// sum runs over the 8 lanes in a fixed tree order, so every workgroup gets the
// same bits).  Readers need a barrier after it.
__device__ inline void top8_weights(const float* lg, const int (&t)[K], int* sel_e, float* sel_w) {
  const int tid = threadIdx.x;
  if (tid < WAVE) {
    const int j = tid & (K - 1);
    int me = t[0];
#pragma unroll
    for (int r = 1; r < K; ++r) me = j == r ? t[r] : me;
    const float ex = __expf(lg[me] - lg[t[0]]);
    const float den = sum8(ex);
    int pos = 0;
#pragma unroll
    for (int r = 0; r < K; ++r) pos += t[r] < me;
    if (tid < K) {
      pos = min(pos, K - 1);
      sel_e[pos] = me;
      sel_w[pos] = ex * __builtin_amdgcn_rcpf(den);
    }
  }
}

}  // namespace dec
}  // namespace moe
