// Expert FFN on MFMA for few routed rows per expert (a decode batch: 32 tokens
// x top-8 over 128 experts gives ~7 rows per active expert).  Same two stages
// and the same operands as the grouped GEMM (grouped_gemm.hip): activations as
// fp16 planes, weights as exact integer codes with the block scale applied per
// block after the MFMA (mfma_frag.hpp), fp32 accumulation.
//
// With so few rows the grouped GEMM's tiles (256 weight rows, a K loop of
// 64-value chunks two deep) are few and latency-bound.  Here the weight slice
// is the unit of work: an item is one 16-row unit of an active expert's routed
// rows (an expert with 7 rows is one unit, one with 17-32 rows two) and a slice
// of the expert's weight rows (gate/up: 16 gate + 16 up rows = 16 columns of h;
// down: 64 rows).  The workgroup copies the whole slice (K = 2048 or 768) from
// global memory straight into LDS at once (LDS DMA, no registers) and applies
// it to the unit's rows, one M-tile.  Activation fragments come through buffer
// loads; a padding row of the M-tile (7 rows fill 7 of its 16) gets an offset
// past the buffer's range, which returns zeros without fetching.  The four
// wavefronts split K into quarters and add their partial tiles in LDS in
// wavefront order, so the result does not depend on timing.  Weight rows sit in
// LDS with a stride that is an odd multiple of 16 bytes, which puts the 16 rows
// x 4 lane groups of a fragment read in distinct banks.  The grid is
// persistent: every workgroup builds the list of units from expert_offsets (in
// LDS) and takes (unit, slice) items in rounds over the grid.
//
// Why units of one M-tile: a hot expert's 17-32 rows as one two-tile item took
// well over twice a one-tile item (the prefetch ring is half as deep per tile),
// two such items on one CU set the end of the launch, and the two-tile code
// kept the kernel at two workgroups per CU.  With one tile the 4-bit kernels fit
// four workgroups per CU (128 registers, at most 40 KB of LDS), and each CU keeps
// four items' slice copies and dots in flight; the units of a slice read the
// same weight bytes, which the caches serve after the first.
#include "mfma_frag.hpp"

namespace moe {
namespace sk {

using gg::h8;
constexpr int NT = 256;       // 4 wavefronts
constexpr int NW = NT / WAVE;
constexpr int MROWS = 16;     // rows per item (one M-tile)
constexpr int D_TUNED = 2048, F_TUNED = 768;
constexpr int E_MAX = 256;    // experts per layer this kernel takes
constexpr int U_MAX = E_MAX + 512 / 16;   // 16-row units: at most one per expert + one per 16 rows
enum { STAGE_GATEUP = 0, STAGE_DOWN = 1 };

__host__ __device__ constexpr int padded_row(int rb) { return ((rb / 16) % 2 == 0) ? rb + 16 : rb; }

template <int FMT, int STAGE>
struct Geo {
  static constexpr int BB = FMT == MOE_FMT_Q8_0 ? 34 : 18;
  static constexpr int K = STAGE == STAGE_GATEUP ? D_TUNED : F_TUNED;
  static constexpr int N = STAGE == STAGE_GATEUP ? F_TUNED : D_TUNED;   // output columns
  static constexpr int RB = K / QK * BB;          // bytes per stored weight row
  static constexpr int RBP = padded_row(RB);      // LDS row stride
  static constexpr int WR = STAGE == STAGE_GATEUP ? 32 : 64;   // weight rows per workgroup
  static constexpr int NS = WR / 16;              // 16-row n-subtiles
  static constexpr int COLS = STAGE == STAGE_GATEUP ? 16 : 64; // output columns per workgroup
  static constexpr int NCB = N / COLS;            // workgroups per expert
  static constexpr int BPW = K / QK / NW;         // blocks per wavefront
  static constexpr int W_BYTES = WR * RBP;
  static_assert(NW * NS * WAVE * 16 <= W_BYTES, "partial tiles fit in the slice's LDS");
  static_assert(RB % 16 == 0 && (RBP / 16) % 2 == 1, "row stride");
  static_assert(K % (QK * NW) == 0 && N % COLS == 0, "shape");
};

struct Args {
  const _Float16* ahi;
  const _Float16* alo;
  const int32_t* rows;
  const int32_t* offsets;
  int k;
  int a_mode;                 // GG_A_*: activation row of sorted row i
  const uint8_t* w0;          // gate (gate/up stage) or down
  int64_t s0;
  const uint8_t* w1;          // up
  int64_t s1;
  int E, R;
  _Float16* ohi;              // gate/up: h planes [R][N] in sorted order
  _Float16* olo;
  float* y;                   // down: y [R][N] in flat order
};

// The item's rows (nv <= 16 of them real, one M-tile) against this wavefront's
// quarter of K: the wavefront's partial tile of every n-subtile goes to acc.
template <int FMT, int STAGE, bool SPLIT>
__device__ inline void pass_tile(const Args& p, const uint8_t* wl, const int* m_src, int kb0,
                                 int lane, int nv, f32x4 (&acc)[Geo<FMT, STAGE>::NS]) {
  using G = Geo<FMT, STAGE>;
  constexpr int PL = SPLIT ? 2 : 1;
  const int ln = lane % 16, lg = lane / 16;
  // activation rows through buffer loads: a padding row's lanes get an offset past
  // the buffer's range, so the load returns zeros without fetching anything
  constexpr int NREC = 1 << 30;                     // > any activation plane (512 rows x K x 2 bytes)
  const __amdgpu_buffer_rsrc_t rs[2] = {
      __builtin_amdgcn_make_buffer_rsrc((void*)p.ahi, 0, NREC, 0x00020000),
      __builtin_amdgcn_make_buffer_rsrc((void*)p.alo, 0, NREC, 0x00020000)};
  const int voff = ln < nv ? m_src[ln] * G::K * 2 : NREC;
  // activation-fragment prefetch depth (blocks): 4 for the 4-bit gate/up stage, so that
  // it fits 128 registers and four workgroups per CU
  constexpr int PD = (FMT == MOE_FMT_Q4 && STAGE == STAGE_GATEUP) ? 4 : 8;
  h8 ra[PD][PL];                                    // prefetch ring of activation fragments
  auto aload = [&](int j, int slot) {
    const int o = ((kb0 + j) * QK + 8 * lg) * 2;
#pragma unroll
    for (int pl = 0; pl < PL; ++pl)
      ra[slot][pl] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rs[pl], voff + o, 0, 0));
  };
#pragma unroll
  for (int j = 0; j < PD; ++j)
    if (j < G::BPW) aload(j, j);
#pragma unroll
  for (int s = 0; s < G::NS; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < G::BPW; ++j) {
    const int b = kb0 + j, slot = j % PD;
    h8 bq[G::NS];
    float dsc[G::NS];
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
      const uint32_t* rw = (const uint32_t*)(wl + (16 * s + ln) * G::RBP);
      auto rd = [=](int off) { return rw[off >> 2]; };
      bq[s] = gg::frag_codes<FMT>(rd, b, lg);
      dsc[s] = gg::frag_scale<FMT>(rd, b);
    }
    const h8 ah = ra[slot][0];
    h8 al;
    if constexpr (SPLIT) al = ra[slot][1];
    if (j + PD < G::BPW) aload(j + PD, slot);
    // t = (a_hi [+ a_lo]) . q on the exact codes, then acc += d * t (the block's
    // scale of the lane's output column)
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
      f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq[s], zero, 0, 0, 0);
      if constexpr (SPLIT) t = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bq[s], t, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[s][i] = __builtin_fmaf(dsc[s], t[i], acc[s][i]);
    }
  }
}

// (four workgroups per CU for the 4-bit weights, two for Q8_0, whose slice
// takes twice the LDS: each workgroup's slice copy and epilogue are covered by
// the others' dots)
template <int FMT, int STAGE, bool SPLIT>
__global__ __launch_bounds__(NT, FMT == MOE_FMT_Q4 ? 4 : 2) void skinny_kernel(Args p) {
  using G = Geo<FMT, STAGE>;
  __shared__ __attribute__((aligned(16))) uint8_t wl[G::W_BYTES];
  __shared__ int m_src[MROWS];
  __shared__ int m_flat[MROWS];
  __shared__ uint8_t act[U_MAX];                    // 16-row units of experts with rows
  __shared__ int aoff[2 * U_MAX];                   // their row ranges (lo, hi)
  __shared__ int n_act;

  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int ln = lane % 16, lg = lane / 16;

  // ---- units (wavefront 0, in expert order): an expert's rows split into 16-row
  // units, so every item is one M-tile ----
  if (wave == 0) {
    int base = 0;
    for (int e0 = 0; e0 < p.E; e0 += WAVE) {
      const int e = e0 + lane;
      int lo = 0, hi = 0;
      if (e < p.E) {
        lo = min(max(p.offsets[e], 0), p.R);
        hi = min(max(p.offsets[e + 1], lo), p.R);
      }
      const int nm = (hi - lo + 15) / 16;
      int incl = nm;
#pragma unroll
      for (int off = 1; off < WAVE; off <<= 1) {
        const int t = __shfl_up(incl, off, WAVE);
        if (lane >= off) incl += t;
      }
      const int pos = base + incl - nm;
      for (int m = 0; m < nm; ++m) {
        act[pos + m] = e;
        aoff[2 * (pos + m)] = lo + 16 * m;
        aoff[2 * (pos + m) + 1] = min(lo + 16 * (m + 1), hi);
      }
      base += __shfl(incl, WAVE - 1, WAVE);
    }
    if (lane == 0) n_act = base;
  }
  __syncthreads();
  const int items = n_act * G::NCB;
  const int kb0 = wave * G::BPW;                    // this wavefront's first block

  // Items go out in rounds over the grid, every other round to its first half
  // only: the first workgroups dispatched (one or two per CU) are the oldest on
  // their CU and issue first, so they finish items sooner than the CU's later ones
  // (an even walk left those last by ~10 us).
  int base = 0;
  for (int r = 0; base < items; ++r) {
    const int width = r % 2 == 1 ? max((int)gridDim.x / 2, 1) : (int)gridDim.x;
    const int it = base + (int)blockIdx.x;
    base += width;
    if ((int)blockIdx.x >= width || it >= items) continue;   // uniform over the workgroup
    const int u = it / G::NCB, cb = it % G::NCB;
    const int e = act[u], r0 = aoff[2 * u], r1 = aoff[2 * u + 1], re = r1 - r0;

    // ---- the weight slice, all of it in flight at once, straight into LDS: wavefront
    // w copies rows w, w + 4, ... (a row's RB/16 pieces in 64-lane instructions, so
    // the padded row stride is kept) ----
    const int n0 = cb * (STAGE == STAGE_GATEUP ? 16 : G::COLS);
    const int es = __builtin_amdgcn_readfirstlane(e), ns = __builtin_amdgcn_readfirstlane(n0);
    for (int row = __builtin_amdgcn_readfirstlane(wave); row < G::WR; row += NW) {
      const uint8_t* src;
      if constexpr (STAGE == STAGE_GATEUP)
        src = row < 16 ? p.w0 + (int64_t)es * p.s0 + (int64_t)(ns + row) * G::RB
                       : p.w1 + (int64_t)es * p.s1 + (int64_t)(ns + row - 16) * G::RB;
      else
        src = p.w0 + (int64_t)es * p.s0 + (int64_t)(ns + row) * G::RB;
#pragma unroll
      for (int c0 = 0; c0 < G::RB / 16; c0 += WAVE)
        if (c0 + lane < G::RB / 16) gg::lds_dma16(src, 16u * (c0 + lane), wl + row * G::RBP + 16 * c0);
    }

    {
      if (tid < MROWS) {
        const int i = r0 + tid;
        int src = 0, fl = -1;
        if (i < r1) {
          const int f = p.rows[i];
          if ((unsigned)f < (unsigned)p.R) {
            fl = f;
            src = p.a_mode == GG_A_TOKEN ? f / p.k : (p.a_mode == GG_A_FLAT ? f : i);
          }
        }
        m_src[tid] = src;
        m_flat[tid] = fl;
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wavefront's slice rows
      __syncthreads();                                // the slice and row metadata
      f32x4 acc[G::NS];
      pass_tile<FMT, STAGE, SPLIT>(p, wl, m_src, kb0, lane, re, acc);

      // ---- K quarters summed in wavefront order, four rows per wavefront ----
      // The partial tiles go to the slice's LDS (free once every wavefront has passed
      // over it).  Wavefront w then takes rows 4w .. 4w+3: its lane (c, i) holds
      // element i of lane c + 16w of each wavefront's partial, i.e. row 4w + i,
      // column c, and adds the four in wavefront order.
      __syncthreads();                                // every wavefront is done with the slice
      f32x4* rd = (f32x4*)wl;
#pragma unroll
      for (int s = 0; s < G::NS; ++s) rd[(wave * G::NS + s) * WAVE + lane] = acc[s];
      __syncthreads();
      {
        const int c = lane % 16, i = lane / 16, r = 4 * wave + i;
        float v[G::NS];
#pragma unroll
        for (int s = 0; s < G::NS; ++s) {
          v[s] = rd[s * WAVE + c + 16 * wave][i];
#pragma unroll
          for (int w = 1; w < NW; ++w) v[s] += rd[(w * G::NS + s) * WAVE + c + 16 * wave][i];
        }
        const int fl = m_flat[r];
        if (fl >= 0) {                                // else a padding row
          if constexpr (STAGE == STAGE_GATEUP) {
            const int64_t o = (int64_t)(r0 + r) * G::N + plane_pos(n0 + c);
            const float hv = silu(v[0]) * v[1];
            const _Float16 hh = (_Float16)hv;
            p.ohi[o] = hh;
            if constexpr (SPLIT) p.olo[o] = (_Float16)(hv - (float)hh);
          } else {
            float* yrow = p.y + (int64_t)fl * G::N + n0 + c;
#pragma unroll
            for (int s = 0; s < G::NS; ++s) yrow[16 * s] = v[s];
          }
        }
      }
      __syncthreads();                                // metadata, partials and the slice reused
    }
  }
}

// Resident workgroups of a kernel on the current device (cached), 0 on failure.
template <typename Kern>
static int resident(Kern k, int slot) {
  static int cache[64][8];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || slot < 0 || slot >= 8) return 0;
  if (cache[dev][slot] == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, NT, 0) != hipSuccess || per <= 0)
      return 0;
    cache[dev][slot] = cus * per;
  }
  return cache[dev][slot];
}

template <int FMT, int STAGE, bool SPLIT>
static hipError_t launch_t(const Args& a, hipStream_t s) {
  using G = Geo<FMT, STAGE>;
  auto k = skinny_kernel<FMT, STAGE, SPLIT>;
  const int slot = FMT * 4 + STAGE * 2 + (SPLIT ? 1 : 0);
  int grid = resident(k, slot);
  if (grid <= 0) return hipErrorInvalidDevice;
  const int items = a.E * G::NCB;                   // upper bound of the item count
  if (grid > items) grid = items;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int FMT, int STAGE>
static hipError_t launch_f(const Args& a, bool split, hipStream_t s) {
  return split ? launch_t<FMT, STAGE, true>(a, s) : launch_t<FMT, STAGE, false>(a, s);
}

}  // namespace sk

bool skinny_supported(const ExpertsDev& W, int64_t R, bool need_gate_up) {
  if (W.D != sk::D_TUNED || W.F != sk::F_TUNED || R > 512 || W.E > sk::E_MAX) return false;
  if (W.fmt != MOE_FMT_Q8_0 && W.fmt != MOE_FMT_Q4) return false;
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!a16(W.down) || (W.down_stride & 15)) return false;
  if (need_gate_up && (!a16(W.gate) || !a16(W.up) || (W.gate_stride & 15) || (W.up_stride & 15)))
    return false;
  return true;
}

hipError_t launch_skinny_gateup(const _Float16* xhi, const _Float16* xlo, int a_mode,
                                const ExpertsDev& W, const int32_t* offsets, const int32_t* rows,
                                int64_t R, int k, _Float16* hhi, _Float16* hlo, bool split,
                                hipStream_t s) {
  if (R <= 0) return hipSuccess;
  sk::Args p{};
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
  p.ohi = hhi;
  p.olo = hlo;
  return W.fmt == MOE_FMT_Q8_0 ? sk::launch_f<MOE_FMT_Q8_0, sk::STAGE_GATEUP>(p, split, s)
                               : sk::launch_f<MOE_FMT_Q4, sk::STAGE_GATEUP>(p, split, s);
}

hipError_t launch_skinny_down(const _Float16* hhi, const _Float16* hlo, int a_mode,
                              const ExpertsDev& W, const int32_t* offsets, const int32_t* rows,
                              int64_t R, int k, float* y, bool split, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  sk::Args p{};
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
  p.y = y;
  return W.fmt == MOE_FMT_Q8_0 ? sk::launch_f<MOE_FMT_Q8_0, sk::STAGE_DOWN>(p, split, s)
                               : sk::launch_f<MOE_FMT_Q4, sk::STAGE_DOWN>(p, split, s);
}

}  // namespace moe
