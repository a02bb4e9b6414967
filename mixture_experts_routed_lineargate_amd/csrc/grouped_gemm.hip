// Grouped GEMM over per-expert row groups on MFMA (gfx950): the batched and
// prefill expert FFN.  The rows routed to expert e are the contiguous range
// expert_offsets[e] .. expert_offsets[e+1] of sorted_rows (the compact
// per-expert grouping of the reuse-ordering page, "What changed from the first
// experiment": the down projection runs over the existing grouping without a
// new routing sort).  Two stages:
//
//   gate/up  h[i][f] = silu(a_i . Wg_e[:, f]) * (a_i . Wu_e[:, f])   (K = d_model)
//   down     y[i][n] = a_i . Wd_e[:, n]                              (K = d_ff)
//            combined as out[t][n] += w_{t,j} y[i][n] (fp32 atomics), or
//            stored as y[flat][n] for an ordered combine.
//
// Tiles.  A workgroup (4 wavefronts) owns BM = 16*MSUB rows of one expert and
// 128 weight rows (down: 128 output columns; gate/up: 64 gate + 64 up rows of
// the same 64 columns of h, so the SwiGLU epilogue is lane-local).  The tile
// list is not materialised: each workgroup reads expert_offsets, scans the
// per-expert tile counts in one wavefront and finds its own (expert, M-tile,
// N-tile), so the grid is sized for the worst case and surplus workgroups exit
// at once.  Workgroups are numbered so that consecutive tiles (the N-tiles of
// one M-tile, then the next M-tile of the same expert) land on the same XCD
// (dispatch is round-robin over the 8 XCDs), where they share activation rows
// and weight tiles through that XCD's L2.
//
// K loop: chunks of 4 blocks (128 values).  Each chunk of activations (fp32)
// and raw weight blocks is prefetched into registers while the previous chunk
// is multiplied, then written to LDS: activations as fp16 (x = hi + lo with two
// fp16 terms unless the single-rounding variant is asked for), weight blocks
// byte-for-byte.  Weights enter the MFMA as exact small integers (q for Q8_0,
// q - 8 for 4-bit, both exact in fp16) built with the 0x6400 exponent trick;
// one v_mfma_f32_16x16x32_f16 covers exactly one 32-value block, and its fp32
// result is scaled by that block's fp16 scale into the fp32 accumulator.  So
// the only roundings are those of the activations (none beyond fp32 with the
// split) and fp32 accumulation.
#include "internal.hpp"

namespace moe {
namespace gg {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;               // threads per workgroup
constexpr int NW = NT / WAVE;         // 4 wavefronts
constexpr int BN = 128;               // weight rows per tile
constexpr int BKB = 4;                // blocks per K chunk
constexpr int BK = BKB * QK;          // 128 values per K chunk
constexpr int AS = BK + 8;            // fp16 per LDS activation row (272 B: conflict-free b128 reads)

enum { STAGE_GATEUP = 0, STAGE_DOWN = 1 };

struct Args {
  const float* a;            // activations fp32, row length K
  const int32_t* rows;       // sorted_rows [R]
  const int32_t* offsets;    // expert_offsets [E+1]
  const float* topk_w;       // [R] flat (t*k + j), OUT_ATOMIC only
  int k;                     // top-k (token = flat / k)
  int a_mode;                // GG_A_*
  const uint8_t* w0;         // gate (gate/up stage) or down
  int64_t s0;
  const uint8_t* w1;         // up (gate/up stage)
  int64_t s1;
  int E, N, K;               // N = output columns (d_ff for gate/up, d_model for down)
  int R;                     // rows (T * k); offsets and rows are clamped to it
  int n_tiles;
  int out_mode;              // GG_OUT_*
  float* h;                  // GG_OUT_H: [R][N] in sorted order
  float* out;                // GG_OUT_ATOMIC: [T][N]
  float* y;                  // GG_OUT_Y: [R][N] in flat order
};

template <int FMT>
struct Fmt {
  static constexpr int BB = FMT == MOE_FMT_Q8_0 ? 34 : 18;
  static constexpr int CB = BKB * BB;          // bytes of one row in one K chunk (136 / 72)
  static constexpr int U8 = CB / 8;            // 8-byte units per row chunk (17 / 9)
  static constexpr int BUNITS = BN * U8;
  static constexpr int BITERS = (BUNITS + NT - 1) / NT;
  static_assert(CB % 8 == 0, "row chunks are 8-byte multiples");
};

__device__ inline int xcd_swizzle(int bid, int total) {
  // bid = 8 s + x runs on XCD x; give XCD x a contiguous range of tiles
  const int x = bid & 7, s = bid >> 3;
  const int q = total >> 3, r = total & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + s;
}

// Rows of expert e, clamped so that bad offsets cannot index outside [0, R).
__device__ inline int group_count(const Args& p, int e) {
  const int b = max(0, p.offsets[e]), en = min(p.R, p.offsets[e + 1]);
  return max(0, en - b);
}

__device__ inline uint32_t lds32(const uint8_t* p, int off) { return *(const uint32_t*)(p + off); }

// Scale of block b of an LDS weight row (fp16 at byte 0 of the block).
template <int FMT>
__device__ inline float block_scale(const uint8_t* row, int b) {
  constexpr int BB = Fmt<FMT>::BB;
  const int ob = b * BB;                               // b*BB = 2b mod 4
  const uint32_t w = lds32(row, ob & ~3);
  const uint16_t bits = (ob & 2) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
  return half_bits_to_float(bits);
}

// The 8 weights k = 8g .. 8g+7 of block b as exact fp16 (q, or q - 8).
template <int FMT>
__device__ inline h8 block_frag(const uint8_t* row, int b, int g) {
  constexpr int BB = Fmt<FMT>::BB;
  union {
    uint32_t u[4];
    h2 p[4];
    h8 v;
  } r;
  if constexpr (FMT == MOE_FMT_Q8_0) {
    const int s = b * BB + 2 + 8 * g;                  // 2 mod 4 when b is even
    uint32_t q0, q1;
    if (s & 2) {
      const uint32_t d0 = lds32(row, s - 2), d1 = lds32(row, s + 2), d2 = lds32(row, s + 6);
      q0 = __builtin_amdgcn_alignbyte(d1, d0, 2);
      q1 = __builtin_amdgcn_alignbyte(d2, d1, 2);
    } else {
      q0 = lds32(row, s);
      q1 = lds32(row, s + 4);
    }
    // two's complement -> biased unsigned, then 0x64uu = 1024 + u as fp16
    q0 ^= 0x80808080u;
    q1 ^= 0x80808080u;
    r.u[0] = __builtin_amdgcn_perm(0x64646464u, q0, 0x04010400u);
    r.u[1] = __builtin_amdgcn_perm(0x64646464u, q0, 0x04030402u);
    r.u[2] = __builtin_amdgcn_perm(0x64646464u, q1, 0x04010400u);
    r.u[3] = __builtin_amdgcn_perm(0x64646464u, q1, 0x04030402u);
    const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};   // 1024 + 128
#pragma unroll
    for (int i = 0; i < 4; ++i) r.p[i] = r.p[i] - bias;
  } else {
    const int s = b * BB + 2 + 4 * g;                  // 2 mod 4 when b is even
    uint32_t n;
    if (s & 2) {
      n = __builtin_amdgcn_alignbyte(lds32(row, s + 2), lds32(row, s - 2), 2);
    } else {
      n = lds32(row, s);
    }
    // byte j holds element 2j (low nibble) and 2j+1 (high nibble)
    const uint32_t lo = n & 0x0f0f0f0fu, hi = (n >> 4) & 0x0f0f0f0fu;
    r.u[0] = __builtin_amdgcn_perm(hi, lo, 0x0c040c00u) | 0x64006400u;
    r.u[1] = __builtin_amdgcn_perm(hi, lo, 0x0c050c01u) | 0x64006400u;
    r.u[2] = __builtin_amdgcn_perm(hi, lo, 0x0c060c02u) | 0x64006400u;
    r.u[3] = __builtin_amdgcn_perm(hi, lo, 0x0c070c03u) | 0x64006400u;
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};   // 1024 + 8
#pragma unroll
    for (int i = 0; i < 4; ++i) r.p[i] = r.p[i] - bias;
  }
  return r.v;
}

template <int FMT, int STAGE, int MSUB, bool SPLIT>
__global__ __launch_bounds__(NT, 2) void grouped_gemm_kernel(Args p) {
  using FF = Fmt<FMT>;
  constexpr int BM = 16 * MSUB;
  constexpr int BS = FF::CB;                        // LDS bytes per weight row
  __shared__ __attribute__((aligned(16))) _Float16 a_hi[BM * AS];
  __shared__ __attribute__((aligned(16))) _Float16 a_lo[SPLIT ? BM * AS : 8];
  __shared__ __attribute__((aligned(16))) uint8_t bw[BN * BS + 16];   // +16: aligned reads may pass the end
  __shared__ int tstart[MAX_E + 1];
  __shared__ int arow[BM];
  __shared__ int flat[BM];
  __shared__ int tile_info[4];

  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int E = p.E;

  // ---- tile map: scan of ceil(count_e / BM) over experts (wavefront 0) ----
  if (wave == 0) {
    const int per = (E + WAVE - 1) / WAVE;
    const int e0 = lane * per;
    int loc = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) loc += (group_count(p, e) + BM - 1) / BM;
    }
    int inc = loc;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
      const int v = __shfl_up(inc, o, WAVE);
      if (lane >= o) inc += v;
    }
    int run = inc - loc;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        tstart[e] = run;
        run += (group_count(p, e) + BM - 1) / BM;
      }
    }
    if (lane == WAVE - 1) tile_info[0] = inc;
  }
  __syncthreads();
  const int total_m = tile_info[0];
  const int total = total_m * p.n_tiles;
  if ((int)blockIdx.x >= total) return;              // uniform over the workgroup
  const int L = xcd_swizzle(blockIdx.x, total);
  const int mg = L / p.n_tiles, nt = L % p.n_tiles;
  // expert = last e with tstart[e] <= mg (empty experts share the next start)
  int lo_e = 0, hi_e = E - 1;
  while (lo_e < hi_e) {
    const int mid = (lo_e + hi_e + 1) >> 1;
    if (tstart[mid] <= mg) lo_e = mid; else hi_e = mid - 1;
  }
  const int e = lo_e;
  const int row0 = max(0, p.offsets[e]) + (mg - tstart[e]) * BM;
  const int nrows = min(BM, min(p.offsets[e + 1], p.R) - row0);

  if (tid < BM) {
    int ar = -1, fl = -1;
    if (tid < nrows) {
      const int i = row0 + tid;
      fl = p.rows[i];
      if ((unsigned)fl >= (unsigned)p.R) fl = -1;     // not a valid flat index: padding row
      else ar = p.a_mode == GG_A_TOKEN ? fl / p.k : (p.a_mode == GG_A_FLAT ? fl : i);
    }
    arow[tid] = ar;
    flat[tid] = fl;
  }

  // weight rows of this tile
  const int64_t RB = (int64_t)(p.K / QK) * FF::BB;  // bytes per stored weight row
  const uint8_t* wbase0;
  const uint8_t* wbase1;
  int n0;
  if constexpr (STAGE == STAGE_GATEUP) {
    n0 = nt * (BN / 2);
    wbase0 = p.w0 + (int64_t)e * p.s0 + (int64_t)n0 * RB;
    wbase1 = p.w1 + (int64_t)e * p.s1 + (int64_t)n0 * RB;
  } else {
    n0 = nt * BN;
    wbase0 = p.w0 + (int64_t)e * p.s0 + (int64_t)n0 * RB;
    wbase1 = wbase0;
  }
  __syncthreads();

  constexpr int AITERS = BM * (BK / 4) / NT;         // float4 per thread per chunk
  static_assert(AITERS * NT == BM * (BK / 4), "activation chunk split");
  float4 ar_[AITERS];
  u32x2 br_[FF::BITERS];

  auto load_chunk = [&](int c) {
#pragma unroll
    for (int it = 0; it < AITERS; ++it) {
      const int idx = it * NT + tid;
      const int r = idx / (BK / 4), c4 = idx % (BK / 4);
      const int src = arow[r];
      ar_[it] = src >= 0 ? *(const float4*)(p.a + (int64_t)src * p.K + c * BK + 4 * c4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int it = 0; it < FF::BITERS; ++it) {
      const int idx = it * NT + tid;
      if (idx < FF::BUNITS) {
        const int r = idx / FF::U8, u = idx % FF::U8;
        const uint8_t* src;
        if constexpr (STAGE == STAGE_GATEUP)
          src = (r < BN / 2 ? wbase0 + (int64_t)r * RB : wbase1 + (int64_t)(r - BN / 2) * RB);
        else
          src = wbase0 + (int64_t)r * RB;
        br_[it] = __builtin_nontemporal_load((const u32x2*)(src + c * FF::CB + 8 * u));
      }
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int it = 0; it < AITERS; ++it) {
      const int idx = it * NT + tid;
      const int r = idx / (BK / 4), c4 = idx % (BK / 4);
      const float v[4] = {ar_[it].x, ar_[it].y, ar_[it].z, ar_[it].w};
      _Float16 hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = (_Float16)v[i];
        lo[i] = (_Float16)(v[i] - (float)hi[i]);
      }
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      *(h4*)(a_hi + r * AS + 4 * c4) = h4{hi[0], hi[1], hi[2], hi[3]};
      if constexpr (SPLIT) *(h4*)(a_lo + r * AS + 4 * c4) = h4{lo[0], lo[1], lo[2], lo[3]};
    }
#pragma unroll
    for (int it = 0; it < FF::BITERS; ++it) {
      const int idx = it * NT + tid;
      if (idx < FF::BUNITS) {
        const int r = idx / FF::U8, u = idx % FF::U8;
        *(u32x2*)(bw + r * BS + 8 * u) = br_[it];
      }
    }
  };

  // wavefront w: n-subtile s uses tile weight rows wrow(s) + lane % 16
  int wrow[2];
  if constexpr (STAGE == STAGE_GATEUP) {
    wrow[0] = wave * 16;                   // gate columns n0 + 16w ..
    wrow[1] = BN / 2 + wave * 16;          // up rows of the same columns
  } else {
    wrow[0] = wave * 32;
    wrow[1] = wave * 32 + 16;
  }
  const int ln = lane % 16, lg = lane / 16;

  f32x4 acc[MSUB][2];
#pragma unroll
  for (int m = 0; m < MSUB; ++m)
#pragma unroll
    for (int s = 0; s < 2; ++s) acc[m][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = p.K / BK;
  load_chunk(0);
  for (int c = 0; c < nchunks; ++c) {
    store_chunk();
    __syncthreads();
    if (c + 1 < nchunks) load_chunk(c + 1);
#pragma unroll
    for (int b = 0; b < BKB; ++b) {
      h8 bf[2];
      float sc[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint8_t* row = bw + (wrow[s] + ln) * BS;
        bf[s] = block_frag<FMT>(row, b, lg);
        sc[s] = block_scale<FMT>(row, b);
      }
#pragma unroll
      for (int m = 0; m < MSUB; ++m) {
        const int aoff = (m * 16 + ln) * AS + b * QK + 8 * lg;
        const h8 ahi = *(const h8*)(a_hi + aoff);
        h8 alo;
        if constexpr (SPLIT) alo = *(const h8*)(a_lo + aoff);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bf[s], f32x4{0.f, 0.f, 0.f, 0.f},
                                                              0, 0, 0);
          if constexpr (SPLIT) part = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bf[s], part, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][s][i] = fmaf(part[i], sc[s], acc[m][s][i]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 16m + 4*lg + i, column ln of each n-subtile ----
#pragma unroll
  for (int m = 0; m < MSUB; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m * 16 + 4 * lg + i;
      if (r >= nrows || flat[r] < 0) continue;
      if constexpr (STAGE == STAGE_GATEUP) {
        const int f = n0 + wave * 16 + ln;
        const float g = acc[m][0][i], u = acc[m][1][i];
        p.h[(int64_t)(row0 + r) * p.N + f] = silu(g) * u;
      } else {
        const int fl = flat[r];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int n = n0 + wrow[s] + ln;
          const float v = acc[m][s][i];
          if (p.out_mode == GG_OUT_ATOMIC) {
            const int64_t t = fl / p.k;
            __hip_atomic_fetch_add(p.out + t * p.N + n, p.topk_w[fl] * v, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          } else {
            p.y[(int64_t)fl * p.N + n] = v;
          }
        }
      }
    }
  }
}

// out[i] = residual ? residual[i] : 0 (start value of the atomic combine)
__global__ __launch_bounds__(256) void init_out_kernel(float* __restrict__ out,
                                                       const float* __restrict__ residual,
                                                       int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  ((float4*)out)[i] = residual ? ((const float4*)residual)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int FMT, int STAGE, int MSUB, bool SPLIT>
static hipError_t launch_t(const Args& a, int64_t R, hipStream_t s) {
  constexpr int BM = 16 * MSUB;
  const int64_t max_m = R / BM + (R < a.E ? R : a.E);
  const int64_t grid = max_m * a.n_tiles;
  hipLaunchKernelGGL((grouped_gemm_kernel<FMT, STAGE, MSUB, SPLIT>), dim3((unsigned)grid), dim3(NT),
                     0, s, a);
  return hipGetLastError();
}

template <int FMT, int STAGE>
static hipError_t launch_f(const Args& a, int64_t R, bool small_m, bool split, hipStream_t s) {
  if (small_m)
    return split ? launch_t<FMT, STAGE, 1, true>(a, R, s) : launch_t<FMT, STAGE, 1, false>(a, R, s);
  return split ? launch_t<FMT, STAGE, 4, true>(a, R, s) : launch_t<FMT, STAGE, 4, false>(a, R, s);
}

}  // namespace gg

bool grouped_supported(const ExpertsDev& W, bool need_gate_up) {
  if (W.D % 128 || W.F % 128) return false;
  if (W.fmt != MOE_FMT_Q8_0 && W.fmt != MOE_FMT_Q4) return false;
  auto a8 = [](const void* p) { return ((uintptr_t)p & 7) == 0; };
  if (!a8(W.down) || (W.down_stride & 7)) return false;
  if (need_gate_up && (!a8(W.gate) || !a8(W.up) || (W.gate_stride & 7) || (W.up_stride & 7)))
    return false;
  return true;
}

bool grouped_small_m(int64_t R) { return R <= 2048; }

hipError_t launch_grouped_gateup(const float* a, int a_mode, const ExpertsDev& W,
                                 const int32_t* offsets, const int32_t* rows, int64_t R, int k,
                                 float* h_sorted, bool split, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  gg::Args p{};
  p.a = a;
  p.rows = rows;
  p.offsets = offsets;
  p.k = k;
  p.a_mode = a_mode;
  p.w0 = W.gate;
  p.s0 = W.gate_stride;
  p.w1 = W.up;
  p.s1 = W.up_stride;
  p.E = W.E;
  p.R = (int)R;
  p.N = W.F;
  p.K = W.D;
  p.n_tiles = W.F / (gg::BN / 2);
  p.out_mode = GG_OUT_H;
  p.h = h_sorted;
  const bool sm = grouped_small_m(R);
  return W.fmt == MOE_FMT_Q8_0
             ? gg::launch_f<MOE_FMT_Q8_0, gg::STAGE_GATEUP>(p, R, sm, split, s)
             : gg::launch_f<MOE_FMT_Q4, gg::STAGE_GATEUP>(p, R, sm, split, s);
}

hipError_t launch_grouped_down(const float* a, int a_mode, const ExpertsDev& W,
                               const int32_t* offsets, const int32_t* rows, const float* topk_w,
                               int64_t R, int k, float* out, float* y, bool split, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  gg::Args p{};
  p.a = a;
  p.rows = rows;
  p.offsets = offsets;
  p.topk_w = topk_w;
  p.k = k;
  p.a_mode = a_mode;
  p.w0 = W.down;
  p.s0 = W.down_stride;
  p.E = W.E;
  p.R = (int)R;
  p.N = W.D;
  p.K = W.F;
  p.n_tiles = W.D / gg::BN;
  p.out_mode = out ? GG_OUT_ATOMIC : GG_OUT_Y;
  p.out = out;
  p.y = y;
  const bool sm = grouped_small_m(R);
  return W.fmt == MOE_FMT_Q8_0 ? gg::launch_f<MOE_FMT_Q8_0, gg::STAGE_DOWN>(p, R, sm, split, s)
                               : gg::launch_f<MOE_FMT_Q4, gg::STAGE_DOWN>(p, R, sm, split, s);
}

hipError_t launch_init_out(float* out, const float* residual, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(gg::init_out_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, out,
                     residual, n4);
  return hipGetLastError();
}

}  // namespace moe
