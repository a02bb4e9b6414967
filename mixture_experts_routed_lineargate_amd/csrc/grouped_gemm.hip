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

constexpr int NT = 512;               // threads per workgroup (8 wavefronts, one workgroup per CU)
constexpr int NW = NT / WAVE;
constexpr int BN = 256;               // weight rows per tile (32 per wavefront)
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
  static constexpr int HUNITS = BN / 2 * U8;   // 8-byte units of half a tile's rows
  static constexpr int HITERS = (HUNITS + NT - 1) / NT;
  static_assert(CB % 8 == 0, "row chunks are 8-byte multiples");
};

__device__ inline int xcd_swizzle(int bid, int total) {
  // bid = 8 s + x runs on XCD x; give XCD x a contiguous range of tiles
  const int x = bid & 7, s = bid >> 3;
  const int q = total >> 3, r = total & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + s;
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

constexpr int TW = 8;                  // tiles per metadata window

// Persistent: each workgroup walks tiles L = slot, slot + G, ... where slot()
// gives the workgroups of one XCD consecutive tiles (tiles are numbered M-tile
// major, so an XCD works on a few M-tiles x all their N-tiles at a time and
// shares activation rows and weight tiles in its L2).
//
// Row metadata (activation row, token, combine weight) of a window of TW tiles
// is fetched into LDS in one batch, so the dependent index loads cost one round
// trip per window rather than per tile.  Every load of the K loop is
// unconditional (padding rows read a valid row and are never stored), so the
// compiler's wait counts stay exact and the two-chunk prefetch is not drained.
//
// K pipeline: two register stages and two LDS buffers.  Chunk c+2 is fetched
// while chunk c is multiplied; one barrier per chunk.
template <int FMT, int STAGE, int MSUB, bool SPLIT>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(Args p) {
  using FF = Fmt<FMT>;
  constexpr int BM = 16 * MSUB;
  constexpr int BS = FF::CB;                        // LDS bytes per weight row
  constexpr int A_ELEMS = BM * AS;
  constexpr int B_BYTES = BN * BS + 16;             // +16: aligned reads may pass the end
  static_assert(TW * BM <= NT, "one metadata entry per thread");
  __shared__ __attribute__((aligned(16))) _Float16 a_hi[2][A_ELEMS];
  __shared__ __attribute__((aligned(16))) _Float16 a_lo[2][SPLIT ? A_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint8_t bw[2][B_BYTES];
  __shared__ int offs[MAX_E + 1];                   // expert_offsets clamped to [0, R]
  __shared__ int tstart[MAX_E + 1];                 // M-tiles of experts < e
  __shared__ int total_m;
  __shared__ int m_src[TW][BM];                     // activation row (always a valid row)
  __shared__ int m_flat[TW][BM];                    // flat row t*k+j, -1 = padding
  __shared__ int m_tok[TW][BM];                     // token of the row
  __shared__ float m_w[TW][BM];                     // combine weight of the row

  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int E = p.E;
  for (int e = tid; e <= E; e += NT) offs[e] = min(max(p.offsets[e], 0), p.R);
  __syncthreads();
  if (wave == 0) {
    const int per = (E + WAVE - 1) / WAVE;
    const int e0 = lane * per;
    auto tiles_of = [&](int e) { return (max(offs[e + 1] - offs[e], 0) + BM - 1) / BM; };
    int loc = 0;
    for (int i = 0; i < per; ++i)
      if (e0 + i < E) loc += tiles_of(e0 + i);
    int inc = loc;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
      const int v = __shfl_up(inc, o, WAVE);
      if (lane >= o) inc += v;
    }
    int run = inc - loc;
    for (int i = 0; i < per; ++i)
      if (e0 + i < E) {
        tstart[e0 + i] = run;
        run += tiles_of(e0 + i);
      }
    if (lane == WAVE - 1) total_m = inc;
  }
  __syncthreads();
  const int total = total_m * p.n_tiles;
  const int G = gridDim.x;
#if defined(GG_ORDER_CONTIG)
  // workgroup b takes tiles [b*per, (b+1)*per): the N-tiles of an M-tile run back to back
  // on one CU and share its activation rows through the L2 whatever the dispatch order
  const int per = (total + G - 1) / G;
  const int first = blockIdx.x * per, stride = 1, ntiles = min(per, max(total - first, 0));
#elif defined(GG_ORDER_PLAIN)
  const int first = blockIdx.x, stride = G, ntiles = (total - first + G - 1) / G;
#else
  const int first = xcd_swizzle(blockIdx.x, G), stride = G, ntiles = (total - first + G - 1) / G;
#endif
  const int64_t RB = (int64_t)(p.K / QK) * FF::BB;  // bytes per stored weight row
  const int nchunks = p.K / BK;

  // tile L -> expert e (last e with tstart[e] <= M-tile; empty experts share the
  // next start), first sorted row, rows, N-tile
  auto decode_tile = [&](int L, int& e, int& row0, int& nrows, int& nt) {
    const int mg = L / p.n_tiles;
    nt = L % p.n_tiles;
    int lo_e = 0, hi_e = E - 1;
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) >> 1;
      if (tstart[mid] <= mg) lo_e = mid; else hi_e = mid - 1;
    }
    e = lo_e;
    row0 = offs[e] + (mg - tstart[e]) * BM;
    nrows = min(BM, offs[e + 1] - row0);
  };

  // wavefront w: n-subtile s uses tile weight rows wrow[s] + lane % 16
  int wrow[2];
  if constexpr (STAGE == STAGE_GATEUP) {
    wrow[0] = wave * 16;                   // gate rows: columns n0 + 16w ..
    wrow[1] = BN / 2 + wave * 16;          // up rows of the same columns
  } else {
    wrow[0] = wave * 32;
    wrow[1] = wave * 32 + 16;
  }
  const int ln = lane % 16, lg = lane / 16;

  constexpr int AITERS = BM * (BK / 4) / NT;         // float4 per thread per chunk
  static_assert(AITERS * NT == BM * (BK / 4), "activation chunk split");
  // weight units of a half tile (BN/2 rows): unit j is row j / U8, 8-byte unit j % U8, so
  // consecutive lanes read consecutive bytes; the last partial pass repeats unit HUNITS-1
  int boff[FF::HITERS], bdst[FF::HITERS];
#pragma unroll
  for (int it = 0; it < FF::HITERS; ++it) {
    const int j = min(it * NT + tid, FF::HUNITS - 1);
    boff[it] = (j / FF::U8) * (int)RB + 8 * (j % FF::U8);
    bdst[it] = (j / FF::U8) * BS + 8 * (j % FF::U8);
  }

  for (int k0 = 0; k0 < ntiles; k0 += TW) {
    // ---- metadata of the window's tiles ----
    if (tid < TW * BM) {
      const int w = tid / BM, r = tid % BM;
      const int L = first + (k0 + w) * stride;
      int src = 0, fl = -1, tok = 0;
      float wt = 0.f;
      if (k0 + w < ntiles) {
        int e, row0, nrows, nt;
        decode_tile(L, e, row0, nrows, nt);
        if (r < nrows) {
          const int i = row0 + r;
          const int f = p.rows[i];
          if ((unsigned)f < (unsigned)p.R) {
            fl = f;
            tok = f / p.k;
            src = p.a_mode == GG_A_TOKEN ? tok : (p.a_mode == GG_A_FLAT ? f : i);
            if (p.out_mode == GG_OUT_ATOMIC) wt = p.topk_w[f];
          }
        }
      }
      m_src[w][r] = src;
      m_flat[w][r] = fl;
      m_tok[w][r] = tok;
      m_w[w][r] = wt;
    }
    __syncthreads();

    for (int w = 0; w < TW; ++w) {
      if (k0 + w >= ntiles) break;                    // uniform over the workgroup
      const int L = first + (k0 + w) * stride;
      int e, row0, nrows, nt;
      decode_tile(L, e, row0, nrows, nt);
      int n0;
      const uint8_t* hb0;
      const uint8_t* hb1;
      if constexpr (STAGE == STAGE_GATEUP) {
        n0 = nt * (BN / 2);
        hb0 = p.w0 + (int64_t)e * p.s0 + (int64_t)n0 * RB;          // gate rows
        hb1 = p.w1 + (int64_t)e * p.s1 + (int64_t)n0 * RB;          // up rows
      } else {
        n0 = nt * BN;
        hb0 = p.w0 + (int64_t)e * p.s0 + (int64_t)n0 * RB;
        hb1 = hb0 + (int64_t)(BN / 2) * RB;
      }
      int aoffs[AITERS];
#pragma unroll
      for (int it = 0; it < AITERS; ++it) {
        const int idx = it * NT + tid;
        aoffs[it] = m_src[w][idx / (BK / 4)] * p.K + 4 * (idx % (BK / 4));
      }

      struct Stage {
        float4 a[AITERS];
        u32x2 b[2][FF::HITERS];
      };
      auto load = [&](int c, Stage& st) {
#pragma unroll
        for (int it = 0; it < AITERS; ++it) st.a[it] = *(const float4*)(p.a + aoffs[it] + c * BK);
        const uint8_t* b0 = hb0 + c * FF::CB;
        const uint8_t* b1 = hb1 + c * FF::CB;
#pragma unroll
        for (int it = 0; it < FF::HITERS; ++it) {
          st.b[0][it] = *(const u32x2*)(b0 + boff[it]);
          st.b[1][it] = *(const u32x2*)(b1 + boff[it]);
        }
      };
      auto store = [&](const Stage& st, int buf) {
#pragma unroll
        for (int it = 0; it < AITERS; ++it) {
          const int idx = it * NT + tid;
          const int r = idx / (BK / 4), c4 = idx % (BK / 4);
          const float v[4] = {st.a[it].x, st.a[it].y, st.a[it].z, st.a[it].w};
          _Float16 hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hi[i] = (_Float16)v[i];
            lo[i] = (_Float16)(v[i] - (float)hi[i]);
          }
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          *(h4*)(a_hi[buf] + r * AS + 4 * c4) = h4{hi[0], hi[1], hi[2], hi[3]};
          if constexpr (SPLIT) *(h4*)(a_lo[buf] + r * AS + 4 * c4) = h4{lo[0], lo[1], lo[2], lo[3]};
        }
#pragma unroll
        for (int it = 0; it < FF::HITERS; ++it) {
          *(u32x2*)(bw[buf] + bdst[it]) = st.b[0][it];
          *(u32x2*)(bw[buf] + (BN / 2) * BS + bdst[it]) = st.b[1][it];
        }
      };

      f32x4 acc[MSUB][2];
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s) acc[m][s] = f32x4{0.f, 0.f, 0.f, 0.f};

      auto compute = [&](int buf) {
        const _Float16* ah = a_hi[buf];
        const _Float16* al = a_lo[buf];
        // blocks in pairs (the parity of a block fixes its byte alignment); one pair's
        // fragments live at a time
#pragma unroll 1
        for (int bp = 0; bp < BKB; bp += 2)
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          const int b = bp + b2;
          h8 bf[2];
          float sc[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint8_t* row = bw[buf] + (wrow[s] + ln) * BS;
            bf[s] = block_frag<FMT>(row, b, lg);
            sc[s] = block_scale<FMT>(row, b);
          }
#pragma unroll
          for (int m = 0; m < MSUB; ++m) {
            const int aoff = (m * 16 + ln) * AS + b * QK + 8 * lg;
            const h8 ahi = *(const h8*)(ah + aoff);
            h8 alo;
            if constexpr (SPLIT) alo = *(const h8*)(al + aoff);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  ahi, bf[s], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
              if constexpr (SPLIT)
                part = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bf[s], part, 0, 0, 0);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[m][s][i] = fmaf(part[i], sc[s], acc[m][s][i]);
            }
          }
        }
      };

      // Two stages are always in flight at the loop head (chunk indices are clamped
      // instead of skipping loads), so the compiler's wait counts are exact.
      Stage s0, s1;
      load(0, s0);
      load(min(1, nchunks - 1), s1);
      int c = 0;
      for (; c + 2 < nchunks; c += 2) {
        store(s0, 0);
        __syncthreads();
        load(c + 2, s0);
        compute(0);
        store(s1, 1);
        __syncthreads();
        load(min(c + 3, nchunks - 1), s1);
        compute(1);
      }
      store(s0, 0);                                   // last one or two chunks: no loads
      __syncthreads();
      compute(0);
      if (c + 1 < nchunks) {
        store(s1, 1);
        __syncthreads();
        compute(1);
      }

      // ---- epilogue: lane holds rows 16m + 4*lg + i, column ln of each n-subtile ----
#pragma unroll
      for (int m = 0; m < MSUB; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m * 16 + 4 * lg + i;
          const int fl = m_flat[w][r];
          if (fl < 0) continue;                         // padding row
          if constexpr (STAGE == STAGE_GATEUP) {
            const int f = n0 + wave * 16 + ln;
            const float g = acc[m][0][i], u = acc[m][1][i];
            p.h[(int64_t)(row0 + r) * p.N + f] = silu(g) * u;
          } else if (p.out_mode == GG_OUT_ATOMIC) {
            const float wt = m_w[w][r];
            float* orow = p.out + (int64_t)m_tok[w][r] * p.N + n0 + ln;
#pragma unroll
            for (int s = 0; s < 2; ++s)
              __hip_atomic_fetch_add(orow + wrow[s], wt * acc[m][s][i], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          } else {
            float* yrow = p.y + (int64_t)fl * p.N + n0 + ln;
#pragma unroll
            for (int s = 0; s < 2; ++s) yrow[wrow[s]] = acc[m][s][i];
          }
        }
      }
      __syncthreads();                                  // LDS buffers are reused by the next tile
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

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return -1;
    cache[dev] = cus;
  }
  return cache[dev];
}

template <int FMT, int STAGE, int MSUB, bool SPLIT>
static hipError_t launch_t(const Args& a, int64_t R, hipStream_t s) {
  constexpr int BM = 16 * MSUB;
  const int64_t max_m = R / BM + (R < a.E ? R : a.E);
  int64_t grid = max_m * a.n_tiles;                // upper bound of the tile count
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  if (grid > cus) grid = cus;                       // persistent: one workgroup per CU
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
  // down tiles are 256 columns of d_model; K chunks are 128 values
  if (W.D % 256 || W.F % 128) return false;
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
  p.n_tiles = W.F / (gg::BN / 2);   // 128 columns of h per tile
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
