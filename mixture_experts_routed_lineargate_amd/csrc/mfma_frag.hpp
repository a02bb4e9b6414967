// Weight fragments for v_mfma_f32_16x16x32_f16 built from block-quantized rows
// (shared by the grouped GEMM kernels).  A lane of a B fragment holds the 8
// weights k = 8g .. 8g+7 of one weight row within a 32-value block, as their
// exact integer codes, in the activation planes' order (8g + 0, 2, 4, 6, 1, 3, 5,
// 7: plane_pos), so that the A fragment read from a plane row pairs each code with
// its own activation; the block's fp16 scale is applied to the MFMA result.
// frag_codes / frag_scale read a row staged in LDS through `rd(off)` (the dword
// at byte offset `off`, a multiple of 4, of the stored row); codes_q8 / codes_q4
// turn code dwords into fp16 fragments; lds_dma16 streams 16-byte pieces from
// global memory into LDS.
#pragma once

#include "internal.hpp"

namespace moe {
namespace gg {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

// Eight signed Q8_0 codes b0..b7 (bytes of q0, then q1) as exact fp16 values, in
// the order b0 b2 b4 b6 b1 b3 b5 b7.
__device__ inline h8 codes_q8(uint32_t q0, uint32_t q1) {
  union {
    uint32_t u[4];
    h2 p[4];
    h8 v;
  } r;
  // two's complement -> biased unsigned, then 0x64uu = 1024 + u as fp16
  q0 ^= 0x80808080u;
  q1 ^= 0x80808080u;
  r.u[0] = __builtin_amdgcn_perm(0x64646464u, q0, 0x04020400u);   // b0 b2
  r.u[1] = __builtin_amdgcn_perm(0x64646464u, q1, 0x04020400u);   // b4 b6
  r.u[2] = __builtin_amdgcn_perm(0x64646464u, q0, 0x04030401u);   // b1 b3
  r.u[3] = __builtin_amdgcn_perm(0x64646464u, q1, 0x04030401u);   // b5 b7
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};   // 1024 + 128
#pragma unroll
  for (int i = 0; i < 4; ++i) r.p[i] = r.p[i] - bias;
  return r.v;
}

// Eight 4-bit codes q0..q7 (byte j holds q_2j in its low nibble, q_2j+1 in its
// high nibble) as the exact fp16 values q - 8, in the order q0 q2 q4 q6 q1 q3 q5
// q7: the low nibbles of the four bytes, then the high ones, each pair placed
// under a 0x64 exponent byte by one permute.
__device__ inline h8 codes_q4(uint32_t n) {
  union {
    uint32_t u[4];
    h2 p[4];
    h8 v;
  } r;
  const uint32_t lo = n & 0x0f0f0f0fu, hi = (n >> 4) & 0x0f0f0f0fu;
  r.u[0] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u);   // q0 q2
  r.u[1] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u);   // q4 q6
  r.u[2] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u);   // q1 q3
  r.u[3] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u);   // q5 q7
  const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};   // 1024 + 8
#pragma unroll
  for (int i = 0; i < 4; ++i) r.p[i] = r.p[i] - bias;
  return r.v;
}

// Block b's weights k = 8g .. 8g+7 as exact fp16 codes (q, or q - 8).
template <int FMT, typename Rd>
__device__ inline h8 frag_codes(Rd rd, int b, int g) {
  constexpr int BB = FMT == MOE_FMT_Q8_0 ? 34 : 18;
  if constexpr (FMT == MOE_FMT_Q8_0) {
    const int s = b * BB + 2 + 8 * g;                  // 2 mod 4 when b is even
    uint32_t q0, q1;
    if (s & 2) {
      const uint32_t d0 = rd(s - 2), d1 = rd(s + 2), d2 = rd(s + 6);
      q0 = __builtin_amdgcn_alignbyte(d1, d0, 2);
      q1 = __builtin_amdgcn_alignbyte(d2, d1, 2);
    } else {
      q0 = rd(s);
      q1 = rd(s + 4);
    }
    return codes_q8(q0, q1);
  } else {
    const int s = b * BB + 2 + 4 * g;                  // 2 mod 4 when b is even
    uint32_t n;
    if (s & 2) {
      n = __builtin_amdgcn_alignbyte(rd(s + 2), rd(s - 2), 2);
    } else {
      n = rd(s);
    }
    return codes_q4(n);
  }
}

// Block b's fp16 scale d, as fp32.
template <int FMT, typename Rd>
__device__ inline float frag_scale(Rd rd, int b) {
  constexpr int BB = FMT == MOE_FMT_Q8_0 ? 34 : 18;
  const int ob = b * BB;
  const uint32_t w = rd(ob & ~3);
  const uint16_t bits = (ob & 2) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
  return (float)__builtin_bit_cast(_Float16, bits);
}

// fp16 halves of a dword, as fp32
__device__ inline float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// global_load_lds_dwordx4: lane i of the wavefront writes the 16 bytes at
// base + off (base wavefront-uniform, off a per-lane byte offset below 2^31) to
// LDS bytes lds + 16i .. 16i+15 (lds wavefront-uniform).  Issued from asm so the
// compiler neither orders LDS reads behind it nor counts it: callers wait with an
// explicit vmcnt, or through a later load that completes after it.
__device__ inline void lds_dma16(const void* base, uint32_t off, const uint8_t* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(a)
               : "memory");
}

}  // namespace gg
}  // namespace moe
