// Grouped GEMM over per-expert row groups on MFMA (gfx950): the batched and
// prefill expert FFN.  The rows routed to expert e are the contiguous range
// expert_offsets[e] .. expert_offsets[e+1] of sorted_rows (the compact
// per-expert grouping of the reuse-ordering page, "What changed from the first
// experiment": the down projection runs over the existing grouping without a
// new routing sort).  Two stages:
//
//   gate/up  h[i][f] = silu(a_i . Wg_e[:, f]) * (a_i . Wu_e[:, f])   (K = d_model)
//   down     y[flat][n] = a_i . Wd_e[:, n]                           (K = d_ff)
//
// The weighted combine reads y afterwards in slot order (a plain store of y
// and one pass over it moves fewer bytes per second of GPU time than fp32
// atomic adds into the output: ~13 us of stores plus a read pass, against
// ~50 us for the 16.8M atomics of a 1024-token microbatch), so the result is
// bit-reproducible.
//
// Tiles.  A workgroup (4 wavefronts) owns BM = 16*MSUB rows of one expert and
// 256 weight rows (down: 256 output columns; gate/up: 128 gate + 128 up rows of
// the same 128 columns of h, so the SwiGLU epilogue is lane-local); each
// wavefront computes 64 rows x 64 weight rows.  The tile list is not
// materialised: each workgroup reads expert_offsets, scans the per-expert tile
// counts in one wavefront and walks its own tiles.  Two workgroups share a CU.
//
// Operands.  Activations arrive as fp16 planes (a = hi + lo, or hi alone when
// single rounding is asked for), converted once per call rather than per tile.
// Weights enter the MFMA as their exact integer codes (q, or q - 8 for 4-bit),
// rebuilt as fp16 with the 0x6400 exponent trick.  One MFMA spans one 32-value
// block, so per block t = a_hi . q (+ a_lo . q) comes out of one (two) MFMAs
// with C = 0, and acc += d * t applies the block's fp16 scale: lane (.., ln) of
// a 16x16 accumulator holds output column ln only, so it needs one scale per
// block and n-subtile.  The products are exact; the roundings are those of the
// activations, of fp32 accumulation and of the one FMA per block.  (An exact
// hi/lo fp16 pair for d*q would need three MFMAs per block in split mode and
// twice the dequantisation work; the scaled form is 7-10% faster end to end.)
//
// K loop: chunks of 2 blocks (64 values), both operands streamed from global
// memory straight into LDS (global_load_lds, 16-byte pieces, no registers): the
// activation chunk with its pieces XOR-swizzled by row (conflict-free fragment
// reads), and the tile's 256 weight-row chunks, each copied as whole 16-byte
// pieces into an 80-byte (Q8_0) or 48-byte (4-bit) LDS row from which every lane
// reads its own fragment dwords and block scales.  Two buffers per operand: the
// next chunk is requested while this one is multiplied, then one wait and one
// barrier.  Vector-memory instructions are what bounds this kernel (the
// texture-address unit spends about the same time on every 64-lane load whatever
// its width), and 16-byte pieces need the fewest: per wavefront and chunk 4
// activation and 5 (Q8_0) or 3 (4-bit) weight loads, against 8 weight loads when
// each lane fetched its fragment dwords itself.  A tile whose rows fill fewer than
// four 16-row subtiles multiplies only those.  expert_offsets and the per-expert
// tile starts live in dynamic LDS sized to E, so that the Q8_0 form (77 KB) still
// fits two workgroups per CU.
#include "mfma_frag.hpp"

namespace moe {
namespace gg {

constexpr int NT = 256;               // threads per workgroup (4 wavefronts, two workgroups per CU)
constexpr int BN = 256;               // weight rows per tile (64 per wavefront)
constexpr int BKB = 2;                // blocks per K chunk
constexpr int BK = BKB * QK;          // 64 values per K chunk
// workgroups per CU (at most): two.  Three fit with single-fp16 activations and
// 4-bit weights but measured no faster (the kernel is bound by its VALU work, not
// by waves to hide latency with)
template <bool SPLIT>
constexpr int wg_per_cu() { return 2; }

enum { STAGE_GATEUP = 0, STAGE_DOWN = 1 };

struct Args {
  const _Float16* ahi;       // activations as fp16 planes: a = ahi + alo (alo unused when
  const _Float16* alo;       //   activations are single-rounded), rows of length K
  const int32_t* rows;       // sorted_rows [R]
  const int32_t* offsets;    // expert_offsets [E+1]
  int k;                     // top-k (token = flat / k)
  int a_mode;                // GG_A_*
  const uint8_t* w0;         // gate (gate/up stage) or down
  int64_t s0;
  const uint8_t* w1;         // up (gate/up stage)
  int64_t s1;
  int E, N, K;               // N = output columns (d_ff for gate/up, d_model for down)
  int R;                     // rows (T * k); offsets and rows are clamped to it
  int n_tiles;
  int band;                  // 0: M-tile major; B: N-tiles in bands of B (B divides n_tiles)
  _Float16* ohi;             // gate/up: h planes [R][N] in sorted order
  _Float16* olo;
  float* y;                  // down: y [R][N] in flat order
};

// Weight rows of one K chunk staged in LDS by DMA: a row's chunk (68 / 36 bytes)
// is copied as 16-byte pieces into an LDS row of ROWB bytes; the last piece is
// taken to end exactly at the chunk's end (it overlaps the one before), so no
// read passes the row.
template <int FMT>
struct LdsRow;
template <>
struct LdsRow<MOE_FMT_Q8_0> {
  static constexpr int BB = 34, CB = 2 * BB;       // block bytes; bytes of a row's chunk
  static constexpr int SLOTS = 5, ROWB = 80;
  __device__ static uint32_t piece_off(int j) { return j < 4 ? 16u * j : 52u; }
  // block 0 codes 8g .. 8g+7 (bytes 2+8g ..), block 1 codes (bytes 36+8g ..), scales
  __device__ static void frag(const uint8_t* rb, int g, h8& q0, h8& q1, float& s0, float& s1) {
    const uint32_t* w = (const uint32_t*)rb;
    const uint32_t d0 = w[2 * g], d1 = w[2 * g + 1], d2 = w[2 * g + 2];
    q0 = codes_q8(__builtin_amdgcn_alignbyte(d1, d0, 2), __builtin_amdgcn_alignbyte(d2, d1, 2));
    const uint32_t e0 = w[9 + 2 * g];
    const uint32_t e1 = g < 3 ? w[10 + 2 * g] : w[19];    // bytes 64..67 sit at 76 (last piece)
    q1 = codes_q8(e0, e1);
    s0 = half_lo(w[0]);
    s1 = half_hi(w[8]);
  }
};
template <>
struct LdsRow<MOE_FMT_Q4> {
  static constexpr int BB = 18, CB = 2 * BB;
  static constexpr int SLOTS = 3, ROWB = 48;
  __device__ static uint32_t piece_off(int j) { return j < 2 ? 16u * j : 20u; }
  __device__ static void frag(const uint8_t* rb, int g, h8& q0, h8& q1, float& s0, float& s1) {
    const uint32_t* w = (const uint32_t*)rb;
    q0 = codes_q4(__builtin_amdgcn_alignbyte(w[g + 1], w[g], 2));
    q1 = codes_q4(w[8 + g]);                                 // bytes 20+4g.. sit at 32+4g
    s0 = half_lo(w[0]);
    s1 = half_hi(w[4]);
  }
};

__host__ __device__ constexpr int xcd_swizzle(int bid, int total) {
  // bid = 8 s + x runs on XCD x; give XCD x a contiguous range of tiles
  const int x = bid & 7, s = bid >> 3;
  const int q = total >> 3, r = total & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + s;
}

// The tile walk of a G-workgroup grid over `total` tiles: whole rounds of G
// tiles, workgroup b taking position xcd_swizzle(b, G) in each, then a partial
// round whose positions go first to the older half of the grid (b < G/2).
struct TileWalk {
  int G, first, last, rounds, rest;
  __host__ __device__ constexpr TileWalk(int b, int g, int total)
      : G(g), first(xcd_swizzle(b, g)),
        last(b < g / 2 ? xcd_swizzle(b, g / 2) : g / 2 + xcd_swizzle(b - g / 2, g - g / 2)),
        rounds(total / g), rest(total - total / g * g) {}
  __host__ __device__ constexpr int count() const { return rounds + (last < rest ? 1 : 0); }
  __host__ __device__ constexpr int pos(int k) const { return k < rounds ? first + k * G : rounds * G + last; }
};

// Checked at compile time for the grid sizes below: the walk hands out every
// tile exactly once.
constexpr bool walk_exact(int G, int total) {
  constexpr int CAP = 4096;
  bool seen[CAP] = {};
  if (G < 1 || total < 0 || total > CAP) return false;
  int n = 0;
  for (int b = 0; b < G; ++b) {
    const TileWalk w(b, G, total);
    for (int k = 0; k < w.count(); ++k) {
      const int t = w.pos(k);
      if (t < 0 || t >= total || seen[t]) return false;
      seen[t] = true;
      ++n;
    }
  }
  return n == total;
}
static_assert(walk_exact(1, 0) && walk_exact(1, 5) && walk_exact(2, 3) && walk_exact(3, 7) &&
                  walk_exact(7, 50) && walk_exact(9, 9) && walk_exact(13, 100) &&
                  walk_exact(256, 255) && walk_exact(512, 0) && walk_exact(512, 511) &&
                  walk_exact(512, 513) && walk_exact(512, 1400) && walk_exact(510, 4096) &&
                  walk_exact(1024, 3000) && walk_exact(511, 700) && walk_exact(1023, 2000) &&
                  walk_exact(257, 4096),
              "tile walk");

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

// Persistent: each workgroup walks tiles L = slot, slot + G, ... where slot()
// gives the workgroups of one XCD consecutive tiles (tiles are numbered M-tile
// major, so an XCD works on a few M-tiles x their N-tiles at a time and can
// share activation rows and weight tiles in its L2).
//
// Row metadata (activation row, flat row) of a window of TW tiles is fetched
// into LDS in one batch, so the dependent index loads cost one round trip per
// window rather than per tile.
//
// K pipeline: see the loop below (both operands one chunk ahead in two LDS
// buffers each, one wait and one barrier per 64-value chunk).
//
// Wavefront w computes 64 rows x 64 weight rows (4 x 4 MFMA tiles): down rows
// 64w .. 64w+63, or gate rows 32w .. 32w+31 (subtiles 0, 1) and the up rows
// of the same columns (subtiles 2, 3).  Activation chunks are stored in LDS
// with their 16-byte pieces XOR-swizzled by row, so the 16 rows a fragment
// read touches fall in distinct banks.
template <int FMT, int STAGE, int MSUB, bool SPLIT>
__global__ __launch_bounds__(NT, wg_per_cu<SPLIT>()) void grouped_gemm_kernel(Args p) {
  constexpr int BM = 16 * MSUB;
  constexpr int TW = NT / BM;                       // tiles per metadata window
  constexpr int PL = SPLIT ? 2 : 1;                 // activation planes
  constexpr int A_BYTES = BM * BK * 2;              // one plane of one chunk
  constexpr int A_DMA = BM * (BK / 8) >= NT ? BM * (BK / 8) / NT : 1;   // 16-byte loads / plane
  constexpr int A_SLOTS = BM * (BK / 8);            // 16-byte pieces of one plane of one chunk
  constexpr int BUF = PL * A_BYTES;
  using LR = LdsRow<FMT>;
  constexpr int BBUF = BN * LR::ROWB;               // one chunk of the tile's weight rows
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb[2 * BBUF];
  extern __shared__ int dyn_lds[];                  // 2 (E + 1) ints, sized at launch
  int* offs = dyn_lds;                              // expert_offsets clamped to [0, R]
  int* tstart = dyn_lds + (p.E + 1);                // M-tiles of experts < e
  __shared__ int total_m;
  __shared__ int m_src[TW][BM];                     // activation row (always a valid row)
  __shared__ int m_flat[TW][BM];                    // flat row t*k+j, -1 = padding

  const int tid = threadIdx.x, lane = tid % WAVE;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
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
  // Whole rounds of G tiles, then a partial round (TileWalk).  In a whole round an
  // XCD's workgroups take consecutive tiles.  The partial round goes first to the
  // older half of the grid (blockIdx < G/2, dispatched first, one per CU): a CU
  // issues its older workgroup's waves first, so those finish their tiles sooner.
  const TileWalk walk(blockIdx.x, G, total);
  const int ntiles = walk.count();
  auto wpos = [&](int k) { return walk.pos(k); };
  const int64_t RB = (int64_t)(p.K / QK) * LR::BB;  // bytes per stored weight row
  const int nchunks = p.K / BK;                     // even (K is a multiple of 128)

  auto decode_tile = [&](int L, int& e, int& row0, int& nrows, int& nt) {
    int mg;
    if (p.band > 0) {
      // band bi holds N-tiles bi*band .. +band-1 of every M-tile, M-tile major inside
      const int per_band = total_m * p.band;
      const int bi = L / per_band, r = L % per_band;
      mg = r / p.band;
      nt = bi * p.band + r % p.band;
    } else {
      mg = L / p.n_tiles;
      nt = L % p.n_tiles;
    }
    int lo_e = 0, hi_e = E - 1;                     // last e with tstart[e] <= mg
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) >> 1;
      if (tstart[mid] <= mg) lo_e = mid; else hi_e = mid - 1;
    }
    e = lo_e;
    row0 = offs[e] + (mg - tstart[e]) * BM;
    nrows = min(BM, offs[e + 1] - row0);
  };

  // tile weight row of n-subtile s of this wavefront
  int wrow[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (STAGE == STAGE_GATEUP)
      wrow[s] = (s < 2 ? 0 : BN / 2) + wave * 32 + (s & 1) * 16;
    else
      wrow[s] = wave * 64 + s * 16;
  }
  const int ln = lane % 16, lg = lane / 16;

  for (int k0 = 0; k0 < ntiles; k0 += TW) {
    // ---- metadata of the window's tiles ----
    {
      const int w = tid / BM, r = tid % BM;
      int src = 0, fl = -1;
      if (w < TW && k0 + w < ntiles) {
        int e, row0, nrows, nt;
        decode_tile(wpos(k0 + w), e, row0, nrows, nt);
        if (r < nrows) {
          const int i = row0 + r;
          const int f = p.rows[i];
          if ((unsigned)f < (unsigned)p.R) {
            fl = f;
            src = p.a_mode == GG_A_TOKEN ? f / p.k : (p.a_mode == GG_A_FLAT ? f : i);
          }
        }
      }
      if (w < TW) {
        m_src[w][r] = src;
        m_flat[w][r] = fl;
      }
    }
    __syncthreads();

    for (int w = 0; w < TW; ++w) {
      if (k0 + w >= ntiles) break;                    // uniform over the workgroup
      int e, row0, nrows, nt;
      decode_tile(wpos(k0 + w), e, row0, nrows, nt);
      e = __builtin_amdgcn_readfirstlane(e);          // the tile is the workgroup's: make its
      row0 = __builtin_amdgcn_readfirstlane(row0);    // fields scalar so every address below
      nrows = __builtin_amdgcn_readfirstlane(nrows);  // is a scalar base + lane offset
      nt = __builtin_amdgcn_readfirstlane(nt);
      const int msub = (nrows + 15) / 16;             // 16-row subtiles holding rows
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
      // activation 16-byte pieces of this thread: slot q = i*NT + tid (mod the slots of a
      // plane) is row q / 8, stored piece q % 8, holding logical piece (q % 8) ^ swz(row)
      uint32_t aoff[A_DMA];                           // byte offsets (planes are below 2 GiB)
#pragma unroll
      for (int i = 0; i < A_DMA; ++i) {
        const int q = (i * NT + tid) % (BM * (BK / 8));
        const int r = q / 8, c = (q % 8) ^ ((r >> 1) & 7);
        aoff[i] = ((uint32_t)m_src[w][r] * (uint32_t)p.K + 8u * c) * 2u;
      }
      // Activation chunk c goes straight from global memory into LDS buffer `buf`
      // (global_load_lds: lane i of a wavefront fills bytes 16i .. 16i+15 of the
      // wavefront's 1 KiB destination, so slot q = i*NT + tid lands at 16q).
      // A wavefront's load i covers rows (i*NT + 64*wave) / 8 .. +7; loads that
      // cover only rows past the last 16-row subtile holding rows are skipped
      // (those rows are never multiplied).
      const int arows = ((nrows + 15) / 16) * 16;
      auto load_a = [&](int c, uint8_t* buf) {
        if (A_SLOTS >= NT || wave * WAVE < A_SLOTS) {   // wavefront-uniform
#pragma unroll
          for (int pl = 0; pl < PL; ++pl) {
            const _Float16* src = (pl ? p.alo : p.ahi) + c * BK;
#pragma unroll
            for (int i = 0; i < A_DMA; ++i)
              if ((i * NT + wave * WAVE) / 8 < arows)       // wavefront-uniform
                lds_dma16(src, aoff[i], buf + pl * A_BYTES + (i * NT + wave * WAVE) * 16);
          }
        }
      };

      // Weight rows: wavefront w copies tile rows 64w .. 64w+63 (rows < BN/2 come
      // from hb0, the rest from hb1; BN/2 is a multiple of 64), LR::SLOTS pieces per row.
      const uint8_t* wbase = 64 * wave < BN / 2 ? hb0 + (int64_t)(64 * wave) * RB
                                                 : hb1 + (int64_t)(64 * wave - BN / 2) * RB;
      uint32_t boff[LR::SLOTS];
#pragma unroll
      for (int i = 0; i < LR::SLOTS; ++i) {
        const int q = 64 * i + lane;
        boff[i] = (uint32_t)((q / LR::SLOTS) * RB) + LR::piece_off(q % LR::SLOTS);
      }
      auto load_b = [&](int c, uint8_t* bb) {
#pragma unroll
        for (int i = 0; i < LR::SLOTS; ++i)
          lds_dma16(wbase + (int64_t)c * LR::CB, boff[i], bb + (64 * LR::SLOTS * wave + 64 * i) * 16);
      };

      // The K loop and epilogue of one tile whose rows fill MS 16-row subtiles.
      auto run_tile = [&](auto MSc) {
        constexpr int MS = decltype(MSc)::value;
        f32x4 acc[MS][4];
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[m][s] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Per block: t = (a_hi [+ a_lo]) . q on the exact integer codes, then
        // acc += d * t with the block's fp16 scale d of the lane's column.
        auto compute = [&](const uint8_t* buf, const uint8_t* bb) {
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          h8 bq[BKB][4];
          float dsc[BKB][4];
#pragma unroll
          for (int s = 0; s < 4; ++s) LR::frag(bb + (wrow[s] + ln) * LR::ROWB, lg, bq[0][s], bq[1][s], dsc[0][s], dsc[1][s]);
#pragma unroll
          for (int m = 0; m < MS; ++m) {
            h8 ah[BKB], al[BKB];
            const int r = m * 16 + ln;
#pragma unroll
            for (int b = 0; b < BKB; ++b) {
              const int o = r * (BK * 2) + ((((QK / 8) * b + lg) ^ ((r >> 1) & 7)) * 16);
              ah[b] = *(const h8*)(buf + o);
              if constexpr (SPLIT) al[b] = *(const h8*)(buf + A_BYTES + o);
            }
#pragma unroll
            for (int b = 0; b < BKB; ++b)
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[b], bq[b][s], zero, 0, 0, 0);
                if constexpr (SPLIT) t = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[b], bq[b][s], t, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[m][s][i] = __builtin_fmaf(dsc[b][s], t[i], acc[m][s][i]);
              }
          }
        };

        // One chunk: request the next chunk's activations and weights into the other
        // buffers (freed by the previous chunk), multiply, wait for the requests,
        // one barrier (which publishes them).
        load_a(0, lds);
        load_b(0, ldsb);
        __builtin_amdgcn_s_waitcnt(0x0f70);          // vmcnt(0)
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
          const int bc = c & 1;
          const int cn = min(c + 1, nchunks - 1);
          load_a(cn, lds + (bc ^ 1) * BUF);
          load_b(cn, ldsb + (bc ^ 1) * BBUF);
          compute(lds + bc * BUF, ldsb + bc * BBUF);
          __builtin_amdgcn_s_waitcnt(0x0f70);
          __syncthreads();
        }

        // ---- epilogue: lane holds rows 16m + 4*lg + i, column ln of each n-subtile ----
#pragma unroll
        for (int m = 0; m < MS; ++m) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = m * 16 + 4 * lg + i;
            const int fl = m_flat[w][r];
            if (fl < 0) continue;                       // padding row
            if constexpr (STAGE == STAGE_GATEUP) {
#pragma unroll
              for (int s = 0; s < 2; ++s) {
                const int64_t o = (int64_t)(row0 + r) * p.N + plane_pos(n0 + wave * 32 + s * 16 + ln);
                const float hv = silu(acc[m][s][i]) * acc[m][s + 2][i];
                const _Float16 hh = (_Float16)hv;
                p.ohi[o] = hh;
                if constexpr (SPLIT) p.olo[o] = (_Float16)(hv - (float)hh);
              }
            } else {
              float* yrow = p.y + (int64_t)fl * p.N + n0 + ln;
#pragma unroll
              for (int s = 0; s < 4; ++s) yrow[wrow[s]] = acc[m][s][i];
            }
          }
        }
      };
      if constexpr (MSUB == 1) {
        run_tile(std::integral_constant<int, 1>{});
      } else {
        static_assert(MSUB == 4, "tiles of 16 or 64 rows");
        if (msub == 4) run_tile(std::integral_constant<int, 4>{});
        else if (msub == 3) run_tile(std::integral_constant<int, 3>{});
        else if (msub == 2) run_tile(std::integral_constant<int, 2>{});
        else run_tile(std::integral_constant<int, 1>{});
      }
      __syncthreads();                                  // metadata / buffers reused next
    }
  }
}

// Resident workgroups per CU of one kernel variant at its dynamic LDS size
// (cached per device and E), at most wg_per_cu.
template <int FMT, int STAGE, int MSUB, bool SPLIT>
static int resident_per_cu(int E) {
  static int cache[64][MAX_E + 1];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || E < 1 || E > MAX_E) return 1;
  int& c = cache[dev][E];
  if (c == 0) {
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, grouped_gemm_kernel<FMT, STAGE, MSUB, SPLIT>, NT,
            (size_t)2 * (E + 1) * sizeof(int)) != hipSuccess || per < 1)
      per = 1;
    c = per < wg_per_cu<SPLIT>() ? per : wg_per_cu<SPLIT>();
  }
  return c;
}

template <int FMT, int STAGE, int MSUB, bool SPLIT>
static hipError_t launch_t(const Args& a, int64_t R, hipStream_t s) {
  constexpr int BM = 16 * MSUB;
  const int64_t max_m = R / BM + (R < a.E ? R : a.E);
  int64_t grid = max_m * a.n_tiles;                // upper bound of the tile count
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int W = resident_per_cu<FMT, STAGE, MSUB, SPLIT>(a.E);
  if (grid > (int64_t)cus * W) grid = (int64_t)cus * W;   // persistent: every workgroup resident
  hipLaunchKernelGGL((grouped_gemm_kernel<FMT, STAGE, MSUB, SPLIT>), dim3((unsigned)grid), dim3(NT),
                     (size_t)2 * (a.E + 1) * sizeof(int), s, a);
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
  // down tiles are 256 columns of d_model, gate/up tiles 128 columns of d_ff; K is
  // consumed in pairs of 64-value chunks
  if (W.D % 256 || W.F % 128) return false;
  if (W.fmt != MOE_FMT_Q8_0 && W.fmt != MOE_FMT_Q4) return false;
  auto a8 = [](const void* p) { return ((uintptr_t)p & 7) == 0; };
  if (!a8(W.down) || (W.down_stride & 7)) return false;
  if (need_gate_up && (!a8(W.gate) || !a8(W.up) || (W.gate_stride & 7) || (W.up_stride & 7)))
    return false;
  return true;
}

bool grouped_small_m(int64_t R) { return R <= 2048; }

// The activation planes are addressed with 32-bit byte offsets.
bool grouped_fits(int64_t T, int64_t R, const ExpertsDev& W) {
  const int64_t lim = (int64_t)1 << 31;
  return T * (int64_t)W.D * 2 < lim && R * (int64_t)W.F * 2 < lim && R * (int64_t)W.D * 2 < lim;
}

hipError_t launch_grouped_gateup(const _Float16* xhi, const _Float16* xlo, int a_mode,
                                 const ExpertsDev& W, const int32_t* offsets, const int32_t* rows,
                                 int64_t R, int k, _Float16* hhi, _Float16* hlo, bool split,
                                 hipStream_t s) {
  if (R <= 0) return hipSuccess;
  gg::Args p{};
  p.ahi = xhi;
  p.alo = xlo;
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
  p.ohi = hhi;
  p.olo = hlo;
  const bool sm = grouped_small_m(R);
  return W.fmt == MOE_FMT_Q8_0
             ? gg::launch_f<MOE_FMT_Q8_0, gg::STAGE_GATEUP>(p, R, sm, split, s)
             : gg::launch_f<MOE_FMT_Q4, gg::STAGE_GATEUP>(p, R, sm, split, s);
}

hipError_t launch_grouped_down(const _Float16* hhi, const _Float16* hlo, int a_mode,
                               const ExpertsDev& W, const int32_t* offsets, const int32_t* rows,
                               int64_t R, int k, float* y, bool split, hipStream_t s,
                               bool banded) {
  if (R <= 0) return hipSuccess;
  gg::Args p{};
  p.ahi = hhi;
  p.alo = hlo;
  p.rows = rows;
  p.offsets = offsets;
  p.k = k;
  p.a_mode = a_mode;
  p.w0 = W.down;
  p.s0 = W.down_stride;
  p.E = W.E;
  p.R = (int)R;
  p.N = W.D;
  p.K = W.F;
  p.n_tiles = W.D / gg::BN;
  p.band = (banded && p.n_tiles % 4 == 0) ? 4 : 0;
  p.y = y;
  const bool sm = grouped_small_m(R);
  return W.fmt == MOE_FMT_Q8_0 ? gg::launch_f<MOE_FMT_Q8_0, gg::STAGE_DOWN>(p, R, sm, split, s)
                               : gg::launch_f<MOE_FMT_Q4, gg::STAGE_DOWN>(p, R, sm, split, s);
}

// hi = fp16(v), lo = fp16(v - hi) for n values (n % 8 == 0, 16-byte aligned), each
// group of 8 in the planes' order (plane_pos)
__global__ __launch_bounds__(256) void to_planes_kernel(const float* __restrict__ src, int64_t n8,
                                                        _Float16* __restrict__ hi,
                                                        _Float16* __restrict__ lo) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 v0 = ((const float4*)src)[2 * i], v1 = ((const float4*)src)[2 * i + 1];
  const float a[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  gg::h8 h, l;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    h[plane_pos(k)] = (_Float16)a[k];
    l[plane_pos(k)] = (_Float16)(a[k] - (float)h[plane_pos(k)]);
  }
  ((gg::h8*)hi)[i] = h;
  if (lo) ((gg::h8*)lo)[i] = l;
}

hipError_t launch_to_planes(const float* src, int64_t n, _Float16* hi, _Float16* lo,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(to_planes_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, src, n8,
                     hi, lo);
  return hipGetLastError();
}

}  // namespace moe
