// Attention-side primitives of the warm decode path (technical-overview page,
// "Validated GPU foundation": RMSNorm, grouped per-head Q/K normalization,
// Q/K/V projections, RoPE, request-local F32 KV append; evidence page,
// "GPU-native foundation" card).  Attention itself (scores, softmax, value
// aggregation, output projection) is listed there as still being integrated
// and is not part of this path.
//
// One launch per call (attn_kernel), a workgroup per (20 projection rows, up to
// 8 tokens): 5120 rows make 256 workgroups, one per compute unit, so no unit
// streams twice the bytes of the others.  20 rows do not divide a head, so a
// workgroup's rows may belong to two heads (q, k or v):
//  1  u_t = rmsnorm(x_t) * attn_gain (every workgroup forms the factor of its
//     tokens), then its 20 rows of [q | k | v] = u_t W.  The rows' blocks are
//     staged once in LDS (copied in 16-byte pieces from the aligned piece below
//     the first row, so the rows sit at an even offset) and reused by every
//     token; wavefront w takes rows w and w + 10, lane b of it block b (and
//     b + 64, ...) of the row.  The products are integer: u is turned, block by
//     block, into 22-bit fixed point relative to the block's largest magnitude,
//     held as three 8-bit digit planes (built from registers, 8 lanes a block),
//     and each weight dword meets them in three v_dot4_i32_i8, exact; one fp32
//     combination and the two scales finish the block (the decode kernels'
//     block_dot_dig).  That is half the vector instructions of fp32
//     products of the codes, which left this step bound by the 16-lane SIMDs.
//     A single token streams the Q8_0 matrix once: the projection is HBM-bound.
//  2  v rows go straight to row pos of the v cache.  q and k rows are published
//     to the workspace as 64-bit words (tag << 32 | fp32 bits, agent-scope
//     stores, no fences: a device-scope fence writes back the whole L2 on this
//     chip).  A workgroup first takes a ticket from the per-(token block, head)
//     counter of each q or k head its rows touch; the counters are never reset:
//     call c's tickets are c*g .. c*g+g-1 (g = the workgroups touching the
//     head), so the tag is c + 1 and the workgroup holding the last ticket
//     finishes the head.  It polls the head's words
//     until all carry the tag (the others already hold tickets and wait on
//     nothing, so the wait ends; it is bounded anyway, and a wait that gives up
//     sets the workspace's error word and yields NaN), then: per-head RMSNorm
//     with the shared q or k gain, RoPE (rotate-half pairs, angles
//     pos * theta^(-2i/hd) formed and reduced modulo 2 pi in fp64), q written,
//     k appended at row pos.
//     The sums run in a fixed order, so results are reproducible.
#include "decode_common.hpp"

namespace moe {
namespace at {

constexpr int NT = 640;           // threads of the projection workgroup (10 wavefronts)
constexpr int NW = NT / WAVE;
constexpr int ROWS = 2 * NW;      // weight rows per workgroup (2 per wavefront)
constexpr int TOKS = 8;           // tokens per workgroup

struct Args {
  const float* x;                 // [T][D]
  const float* gain;              // [D]
  const uint8_t* w;               // [N] rows of D/32 blocks
  uint64_t* words;                // [T][N] published q and k rows, tagged (workspace)
  uint32_t* count;                // [ceil(T/8)][Hq + Hkv] tickets per head (workspace)
  uint32_t* err;                  // error word (workspace byte 64)
  const float* q_gain;            // [hd]
  const float* k_gain;            // [hd]
  const int32_t* pos;             // [T]
  float* q;                       // [T][Hq][hd]
  float* k_cache;                 // [max_pos][Hkv][hd]
  float* v_cache;                 // [max_pos][Hkv][hd]
  int64_t T;
  int D, N, Hq, Hkv, hd, max_pos;
  float eps;
  double log_theta;
};

constexpr int DMAX = 3584;                     // largest d_model (20 rows: 76 KB of LDS)
constexpr int XV = DMAX / 4 / NT + 1;          // float4 loads of one token per thread (2)
constexpr int LDS_PAD = 48;                    // leading misalignment (< 16) + reads past a row end

// Per-head RMSNorm with the shared q or k gain, then RoPE, for head `head` of token
// t, by one wavefront once every row of the head carries tag `tag`: lane takes the
// pairs (i, i + hd/2), i = lane, lane + 64.
__device__ inline void finish(const Args& p, int head, int64_t t, uint32_t tag, int lane) {
  const int half = p.hd / 2;
  const uint64_t* hrow = p.words + t * p.N + (int64_t)head * p.hd;
  float v4[4];
  uint32_t budget = dec::SPIN_LIMIT;
  dec::gather_fn<4>([=](int k) {
                      const int i = lane + WAVE * (k >> 1);
                      return hrow + (i < half ? i + (k & 1) * half : 0);   // clamped: a word of the head
                    },
                    tag, p.err, budget, v4);
  float a[2], b[2];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool on = lane + WAVE * j < half;
    a[j] = on ? v4[2 * j] : 0.f;
    b[j] = on ? v4[2 * j + 1] : 0.f;
    ss = fmaf(a[j], a[j], fmaf(b[j], b[j], ss));
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)p.hd + p.eps);
  const bool is_q = head < p.Hq;
  const float* g = is_q ? p.q_gain : p.k_gain;
  const int pt = p.pos[t];
  float* dst = is_q ? p.q + (t * p.Hq + head) * p.hd
                    : (pt >= 0 && pt < p.max_pos
                           ? p.k_cache + ((int64_t)pt * p.Hkv + (head - p.Hq)) * p.hd
                           : nullptr);
  if (!dst) return;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + WAVE * j;
    if (i >= half) break;
    const float na = a[j] * inv * g[i], nb = b[j] * inv * g[i + half];
    // RoPE: angle pos * theta^(-2i/hd), formed and reduced modulo 2 pi in fp64 (so
    // large positions keep it exact), then sine and cosine of the reduced angle
    const double ang = (double)pt * exp(-(2.0 * i / p.hd) * p.log_theta);
    const double two_pi = 6.283185307179586476925286766559;
    const float r = (float)(ang - two_pi * rint(ang / two_pi));
    float sn, c;
    sincosf(r, &sn, &c);
    dst[i] = na * c - nb * sn;
    dst[i + half] = na * sn + nb * c;
  }
}

template <int FMT>
__global__ __launch_bounds__(NT) void attn_kernel(Args p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];   // ROWS * RB + LDS_PAD
  __shared__ __attribute__((aligned(16))) uint8_t dig[DMAX / QK * 96];   // u of the current token as
  __shared__ float2 dscl[DMAX / QK];                                       // digit planes + block scales
  __shared__ float red[NW];
  constexpr int BB = FMT == MOE_FMT_Q8_0 ? 34 : 18;
  constexpr int WV = (ROWS * (DMAX / QK) * 34 + 32 + 16 * NT - 1) / (16 * NT);   // 16-byte loads / thread
  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int D = p.D, nb = D / QK, D4 = D / 4, hd = p.hd, Hqk = p.Hq + p.Hkv;
  const int64_t RB = (int64_t)nb * BB;
  const int n0 = blockIdx.x * ROWS, nr = min(ROWS, p.N - n0);
  const int hA = n0 / hd, hB = (n0 + nr - 1) / hd;    // at most two heads (ROWS <= hd + 4)
  const int64_t t0 = (int64_t)blockIdx.y * TOKS;
  const int nt = (int)min((int64_t)TOKS, p.T - t0);

  // Every load that depends on nothing goes out first, all of them before the
  // first wait: the rows (contiguous; the 16-byte pieces from the one holding
  // their first byte to the one holding their last, all inside the matrix since
  // N * RB is a multiple of 16), the first token and the gain.  Indices are
  // clamped, so the loads are unconditional and the compiler's wait counts stay
  // exact.
  const int64_t b0 = (int64_t)n0 * RB;
  const uint32_t off = (uint32_t)(b0 & 15);           // even: row r starts at LDS byte off + r * RB
  const u32x4* src = (const u32x4*)(p.w + (b0 - off));
  const int n16 = (int)((off + nr * RB + 15) / 16);
  u32x4 wv[WV];
#pragma unroll
  for (int i = 0; i < WV; ++i) wv[i] = __builtin_nontemporal_load(src + min(i * NT + tid, n16 - 1));
  float4 xq[XV], gq[XV];
#pragma unroll
  for (int i = 0; i < XV; ++i) {
    const int c = min(i * NT + tid, D4 - 1);
    xq[i] = ((const float4*)(p.x + t0 * D))[c];
    gq[i] = ((const float4*)p.gain)[c];
  }
  // a ticket per q/k head the rows touch, taken once the loads are out (tickets only
  // order arrivals; nothing waits on them)
  __shared__ uint32_t s_tag[2];
  __shared__ int s_last[2];
  if (tid < 2) {
    const int h = tid ? hB : hA;
    s_last[tid] = 0;
    if (h < Hqk && (tid == 0 || hB != hA)) {
      const uint32_t groups = (uint32_t)(((h + 1) * hd - 1) / ROWS - h * hd / ROWS + 1);
      const uint32_t tk = __hip_atomic_fetch_add(p.count + blockIdx.y * Hqk + h, 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_tag[tid] = tk / groups + 1u;
      s_last[tid] = tk % groups == groups - 1u;
    }
  }
#pragma unroll
  for (int i = 0; i < WV; ++i)
    if (i * NT + tid < n16) ((u32x4*)lds)[i * NT + tid] = wv[i];

  for (int ti = 0; ti < nt; ++ti) {
    if (ti > 0) {
#pragma unroll
      for (int i = 0; i < XV; ++i)
        xq[i] = ((const float4*)(p.x + (t0 + ti) * D))[min(i * NT + tid, D4 - 1)];
    }
    // RMSNorm factor of this token (block reduction), then u = x * inv * gain in LDS
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < XV; ++i)
      if (i * NT + tid < D4)
        ss += (xq[i].x * xq[i].x + xq[i].y * xq[i].y) + (xq[i].z * xq[i].z + xq[i].w * xq[i].w);
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();                                // also: the rows are in LDS
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += red[w];
    const float inv = 1.0f / sqrtf(tot / (float)D + p.eps);
    // digit planes of u, straight from registers: thread tid holds pieces tid and
    // tid + NT (8 pieces of a block on adjacent lanes; D/4 is a multiple of 8, so a
    // block's lanes are all in or all past the end)
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      if (i * NT < D4) {                            // uniform: whole wavefronts call it
        const int c = i * NT + tid;
        const float u[4] = {xq[i].x * inv * gq[i].x, xq[i].y * inv * gq[i].y,
                            xq[i].z * inv * gq[i].z, xq[i].w * inv * gq[i].w};
        dec::act_digits_reg<FMT, 4>(u, c < D4, c, dig, dscl);
      }
    }
    __syncthreads();

    // wavefront w: rows n0 + w and n0 + w + 10 (a row past N reads LDS bytes
    // nothing loaded, inside the allocation, and is dropped); lane b: blocks b,
    // b + 64, ...
    float acc0 = 0.f, acc1 = 0.f;
    for (int b = lane; b < nb; b += WAVE) {
      dec::ActDig d;
      dec::load_dig(dig, dscl, b, d);
      acc0 += dec::block_dot_dig<FMT>(lds, (uint32_t)(off + wave * RB + b * BB), d);
      acc1 += dec::block_dot_dig<FMT>(lds, (uint32_t)(off + (wave + NW) * RB + b * BB), d);
    }
    acc0 = wave_sum(acc0);
    acc1 = wave_sum(acc1);
    if (lane < 2) {
      const int r = wave + lane * NW, n = n0 + r;
      const float acc = lane ? acc1 : acc0;
      const int h = n / hd;
      if (r < nr && h >= Hqk) {
        const int pt = p.pos[t0 + ti];
        if (pt >= 0 && pt < p.max_pos)
          p.v_cache[((int64_t)pt * p.Hkv + (h - Hqk)) * hd + n % hd] = acc;
      } else if (r < nr) {
        dec::publish(p.words + (t0 + ti) * p.N + n, s_tag[h != hA], acc);
      }
    }
    // dig and red are reused by the next token; after the last one a finishing
    // wavefront goes straight to its head (it polls the words, not this workgroup)
    if (ti + 1 < nt) __syncthreads();
  }
  // ---- the holder of a head's last ticket finishes the head ----
  // job j = (head slot j / nt, token j % nt), wavefront w takes jobs w, w + 10
  for (int j = wave; j < 2 * nt; j += NW)
    if (s_last[j / nt]) finish(p, j / nt ? hB : hA, t0 + j % nt, s_tag[j / nt], lane);
}

}  // namespace at

size_t attn_lds_bytes(int D, int fmt) {
  return (size_t)at::ROWS * (D / QK) * block_bytes(fmt) + at::LDS_PAD;
}

size_t attn_count_offset(int64_t T, int N) {
  return 256 + (((size_t)T * (size_t)N * sizeof(uint64_t) + 255) & ~(size_t)255);
}

hipError_t launch_attn_prep(const float* x, int64_t T, int D, const float* attn_gain,
                            const uint8_t* w_qkv, int fmt, int Hq, int Hkv, int hd,
                            const float* q_gain, const float* k_gain, const int32_t* pos,
                            float theta, float eps, float* q, float* k_cache, float* v_cache,
                            int max_pos, void* ws, hipStream_t s) {
  at::Args a{};
  a.x = x;
  a.gain = attn_gain;
  a.w = w_qkv;
  a.N = (Hq + 2 * Hkv) * hd;
  a.err = (uint32_t*)((char*)ws + ERR_WORD_OFF);
  a.words = (uint64_t*)((char*)ws + 256);
  a.count = (uint32_t*)((char*)ws + attn_count_offset(T, a.N));
  a.q_gain = q_gain;
  a.k_gain = k_gain;
  a.pos = pos;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.T = T;
  a.D = D;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.hd = hd;
  a.max_pos = max_pos;
  a.eps = eps;
  a.log_theta = log((double)theta);
  dim3 grid((unsigned)((a.N + at::ROWS - 1) / at::ROWS), (unsigned)((T + at::TOKS - 1) / at::TOKS));
  const size_t lds = attn_lds_bytes(D, fmt);
  if (fmt == MOE_FMT_Q8_0)
    hipLaunchKernelGGL(at::attn_kernel<MOE_FMT_Q8_0>, grid, dim3(at::NT), lds, s, a);
  else
    hipLaunchKernelGGL(at::attn_kernel<MOE_FMT_Q4>, grid, dim3(at::NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace moe
