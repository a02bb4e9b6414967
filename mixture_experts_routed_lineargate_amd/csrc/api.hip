// C ABI of libmoe_mi355x: host-side validation, workspace layout and dispatch.
// Everything here runs on the host; every kernel is enqueued on the caller's
// stream without synchronising.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "internal.hpp"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Workspace carve_workspace(void* base, int64_t T, int D, int F, int E, int k, int flags) {
  Workspace w{};
  const size_t tk = (size_t)T * (size_t)k;
  const int ks = router_ksplit(T, D);
  size_t off = 0;
  char* b = (char*)base;
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w.sync = (uint32_t*)take(SYNC_BYTES);
  w.part_logits = (float*)take((size_t)ks * (size_t)T * E * sizeof(float));
  w.ids = (int32_t*)take(tk * sizeof(int32_t));
  w.w = (float*)take(tk * sizeof(float));
  w.offsets = (int32_t*)take((size_t)(E + 1) * sizeof(int32_t));
  w.rows = (int32_t*)take(tk * sizeof(int32_t));
  w.h = (float*)take(tk * (size_t)F * sizeof(float));
  w.y = (float*)take(tk * (size_t)D * sizeof(float));
  w.xn = (flags & MOE_F_PRENORM) ? (float*)take((size_t)T * D * sizeof(float)) : nullptr;
  w.xp = (_Float16*)take((size_t)T * D * 2 * sizeof(_Float16));
  w.ssq = (float*)take((size_t)ks * (size_t)T * sizeof(float));
  w.inv = (float*)take((size_t)T * sizeof(float));
  w.bytes = off;
  return w;
}

bool trace_enabled() {
  static int on = -1;
  if (on < 0) {
    const char* v = getenv("MOE_TRACE");
    on = (v && v[0] && v[0] != '0') ? 1 : 0;
  }
  return on == 1;
}

void trace(const char* what, int64_t T, int D, int F, int E, int k, int fmt) {
  if (!trace_enabled()) return;
  fprintf(stderr, "[moe] %s T=%lld D=%d F=%d E=%d k=%d fmt=%d\n", what, (long long)T, D, F, E, k,
          fmt);
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static moe_status check_dims(int64_t T, int D, int E, int k) {
  if (T < 0 || D <= 0 || D % QK || E <= 0 || k <= 0 || k > E) return MOE_E_SHAPE;
  if (E > MAX_E || k > MAX_K || D > 16384) return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

static moe_status check_experts(const moe_experts* W) {
  if (!W) return MOE_E_NULLPTR;
  if (W->format != MOE_FMT_Q8_0 && W->format != MOE_FMT_Q4) return MOE_E_FORMAT;
  if (W->d_model <= 0 || W->d_model % QK || W->d_ff <= 0 || W->d_ff % QK || W->num_experts <= 0)
    return MOE_E_SHAPE;
  if (W->d_model > 16384 || W->d_ff > 16384 || W->num_experts > MAX_E) return MOE_E_UNSUPPORTED;
  if (!W->w_down) return MOE_E_NULLPTR;
  if (!aligned(W->w_down, 2) || W->down_stride % 2 || W->down_stride < 0) return MOE_E_ALIGN;
  return MOE_OK;
}

static moe_status check_gate_up(const moe_experts* W) {
  if (!W->w_gate || !W->w_up) return MOE_E_NULLPTR;
  if (!aligned(W->w_gate, 2) || !aligned(W->w_up, 2) || W->gate_stride % 2 || W->up_stride % 2 ||
      W->gate_stride < 0 || W->up_stride < 0)
    return MOE_E_ALIGN;
  return MOE_OK;
}

#define MOE_TRY(expr)                  \
  do {                                 \
    const moe_status st_ = (expr);     \
    if (st_ != MOE_OK) return st_;     \
  } while (0)

#define HIP_TRY(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return MOE_E_HIP; \
  } while (0)

// The byte ranges [a, a + na) and [b, b + nb) share a byte.
static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

// Route into the given outputs (ids / w must be device buffers of T*k).
static moe_status do_route(const float* x, int64_t T, int D, const float* G, const float* bias,
                           int E, int k, int32_t* ids, float* w, const Workspace& ws,
                           hipStream_t s) {
  const int ks = router_ksplit(T, D);
  HIP_TRY(launch_router_partial(x, T, D, G, E, ws.part_logits, ks, s));
  HIP_TRY(launch_topk(ws.part_logits, ks, T, E, bias, k, ids, w, s));
  return MOE_OK;
}

// planes_ready: the FULL stage's input planes are already in ws.xp (made by the
// top-k pass); res_scale: the residual row t is in[t] * res_scale[t].
static moe_status do_ffn(const float* in, int stage, const ExpertsDev& W, const int32_t* ids,
                         const float* w, const int32_t* offsets, const int32_t* rows, int64_t T,
                         int k, float* y, float* out, int flags, const Workspace& ws,
                         hipStream_t s, bool planes_ready = false,
                         const float* res_scale = nullptr) {
  const bool full = stage == MOE_STAGE_FULL;
  const int64_t R = T * k;
  auto a16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15) == 0; };
  if (grouped_supported(W, full) && grouped_fits(T, R, W) && a16(in) && a16(y) && a16(out)) {
    const bool split = !(flags & MOE_F_FP16_ACT);
    const bool skinny = skinny_supported(W, R, full);
    trace(full ? (split ? "ffn grouped mfma gate/up+down (split fp16)"
                        : "ffn grouped mfma gate/up+down (fp16)")
               : (split ? "ffn grouped mfma down (split fp16)" : "ffn grouped mfma down (fp16)"),
          T, W.D, W.F, W.E, k, W.fmt);
    if (skinny) trace("  (weight-slice kernels: few rows per expert)", T, W.D, W.F, W.E, k, W.fmt);
    // activations as fp16 planes (hi, lo): x [T][D] in ws.xp, h [R][F] in the h region
    _Float16* hhi = (_Float16*)ws.h;
    _Float16* hlo = split ? hhi + (size_t)R * W.F : nullptr;
    int a_mode = GG_A_FLAT;
    if (full) {
      _Float16* xhi = ws.xp;
      _Float16* xlo = split ? xhi + (size_t)T * W.D : nullptr;
      if (!planes_ready) HIP_TRY(launch_to_planes(in, T * (int64_t)W.D, xhi, xlo, s));
      if (skinny)
        HIP_TRY(launch_skinny_gateup(xhi, xlo, GG_A_TOKEN, W, offsets, rows, R, k, hhi, hlo, split,
                                     s));
      else
        HIP_TRY(launch_grouped_gateup(xhi, xlo, GG_A_TOKEN, W, offsets, rows, R, k, hhi, hlo,
                                      split, s));
      a_mode = GG_A_SORTED;
    } else {
      HIP_TRY(launch_to_planes(in, R * (int64_t)W.F, hhi, hlo, s));
    }
    const float* res = (full && (flags & MOE_F_RESIDUAL)) ? in : nullptr;
    float* ybuf = y ? y : ws.y;
    if (skinny)
      HIP_TRY(launch_skinny_down(hhi, hlo, a_mode, W, offsets, rows, R, k, ybuf, split, s));
    else
      HIP_TRY(launch_grouped_down(hhi, hlo, a_mode, W, offsets, rows, R, k, ybuf, split, s,
                                  (flags & MOE_F_BANDED) != 0));
    // the grouped kernels write only the rows the grouping kept: the combine skips
    // dropped entries (ids outside [0, E)) and sets their rows of the caller's y to 0
    if (out)
      HIP_TRY(launch_combine(ybuf, w, T, k, W.D, res, out, s, res_scale, ids, W.E, y));
    else
      HIP_TRY(launch_zero_dropped(ids, R, W.E, W.D, y, s));
    return MOE_OK;
  }
  const char* path = full ? "ffn generic gate/up+down" : "ffn generic down";
  trace(path, T, W.D, W.F, W.E, k, W.fmt);
  const float* h = in;
  if (stage == MOE_STAGE_FULL) {
    HIP_TRY(launch_gateup_generic(in, W, ids, T, k, ws.h, s));
    h = ws.h;
  }
  float* ybuf = y ? y : ws.y;
  HIP_TRY(launch_down_generic(h, W, ids, T, k, ybuf, s));
  if (out) {
    const float* res = (stage == MOE_STAGE_FULL && (flags & MOE_F_RESIDUAL)) ? in : nullptr;
    HIP_TRY(launch_combine(ybuf, w, T, k, W.D, res, out, s));
  }
  return MOE_OK;
}

// The body of moe_layer after validation.
static moe_status layer_impl(const float* x, const float* gate, const float* bias,
                             const moe_experts* W, int64_t T, int k, int flags, float* out,
                             int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                             int32_t* sorted_rows, void* ws, hipStream_t s) {
  const int D = W->d_model, F = W->d_ff, E = W->num_experts;
  const Workspace w = carve_workspace(ws, T, D, F, E, k, flags);
  const ExpertsDev dev = to_dev(*W);
  int32_t* ids = topk_ids ? topk_ids : w.ids;
  float* wts = topk_w ? topk_w : w.w;
  int32_t* offs = expert_offsets ? expert_offsets : w.offsets;
  int32_t* rows = sorted_rows ? sorted_rows : w.rows;
  if (T == 1 && decode_stack_layer_ok(dev, k) && decode_stack_io_ok(x, out)) {
    // one token: the decode stack kernel with one layer
    trace("layer fused decode", T, D, F, E, k, W->format);
    const StackLayer sl{gate, bias, dev};
    HIP_TRY(launch_decode_stack(x, 1, &sl, dev.fmt, (flags & MOE_F_PRENORM) != 0,
                                (flags & MOE_F_RESIDUAL) != 0, out, topk_ids, topk_w,
                                expert_offsets, sorted_rows, w, s));
    return MOE_OK;
  }
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (grouped_supported(dev, true) && grouped_fits(T, T * k, dev) && a16(x) && a16(out) &&
      D % 4 == 0) {
    // MFMA path: the router also sums x^2 per slice; the top-k pass forms the
    // RMSNorm factor, the routing, and the fp16 planes of the normalised input, so
    // neither a normalisation pass nor a separate conversion pass runs
    trace("layer grouped (fused norm + planes)", T, D, F, E, k, W->format);
    const bool pre = (flags & MOE_F_PRENORM) != 0;
    const bool split = !(flags & MOE_F_FP16_ACT);
    _Float16* xlo = split ? w.xp + (size_t)T * D : nullptr;
    if (route_small_supported(T, D, E, k)) {
      // small batch: router, top-k and grouping in one launch
      HIP_TRY(launch_route_small(x, T, D, gate, bias, E, k, pre, ids, wts, pre ? w.inv : nullptr,
                                 w.xp, xlo, offs, rows, w, s));
    } else {
      const int ks = router_ksplit(T, D);
      HIP_TRY(launch_router_partial(x, T, D, gate, E, w.part_logits, ks, s, pre ? w.ssq : nullptr));
      TopkExtra ex;
      ex.ssq = pre ? w.ssq : nullptr;
      ex.D = D;
      ex.inv = pre ? w.inv : nullptr;
      ex.x = x;
      ex.xhi = w.xp;
      ex.xlo = xlo;
      HIP_TRY(launch_topk(w.part_logits, ks, T, E, bias, k, ids, wts, s, ex));
      HIP_TRY(launch_group(ids, T * k, E, offs, rows, s));
    }
    return do_ffn(x, MOE_STAGE_FULL, dev, ids, wts, offs, rows, T, k, nullptr, out,
                  flags & (MOE_F_RESIDUAL | MOE_F_DETERMINISTIC | MOE_F_FP16_ACT | MOE_F_BANDED), w, s,
                  /*planes_ready=*/true, pre ? w.inv : nullptr);
  }
  trace("layer generic", T, D, F, E, k, W->format);
  const float* u = x;
  if (flags & MOE_F_PRENORM) {
    HIP_TRY(launch_rmsnorm(x, T, D, PRENORM_EPS, w.xn, s));
    u = w.xn;
  }
  MOE_TRY(do_route(u, T, D, gate, bias, E, k, ids, wts, w, s));
  HIP_TRY(launch_group(ids, T * k, E, offs, rows, s));
  return do_ffn(u, MOE_STAGE_FULL, dev, ids, wts, offs, rows, T, k, nullptr, out,
                flags & (MOE_F_RESIDUAL | MOE_F_DETERMINISTIC | MOE_F_FP16_ACT | MOE_F_BANDED), w, s);
}

// ---- the allocation-free variant of moe_layer ----
// Its workspace is this file-scope device array (one copy per GPU, held until the
// process ends).  In host code `scratch` names a host-side stand-in, not a device
// address: the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that pointer is used from then on.
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];
static void* scratch_dev[64];            // per-device address of `scratch`
static std::mutex scratch_mu;

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The device address of the current device's scratch array.  The first call on a
// device looks it up and enqueues, on `s` ahead of the caller's work, a zero fill of
// the exchange region (launch counters and tagged words must start at zero); a
// fill kernel rather than a memset, so that a call captured in a graph replays it
// correctly.
static moe_status scratch_for_device(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_E_HIP;
  if (dev < 0 || dev >= 64) return MOE_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_E_HIP;
    static_assert(SYNC_BYTES % 16 == 0 && SYNC_BYTES <= NOALLOC_SCRATCH_BYTES, "fill size");
    hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, s, (uint4*)p,
                       (size_t)SYNC_BYTES / 16);
    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_NULLPTR: return "required pointer is NULL";
    case MOE_E_SHAPE: return "invalid shape";
    case MOE_E_ALIGN: return "misaligned pointer or stride";
    case MOE_E_FORMAT: return "unknown block format or stage";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_UNSUPPORTED: return "shape outside supported limits";
    case MOE_E_HIP: return "HIP launch failed";
    case MOE_E_TIMEOUT: return "a bounded exchange wait gave up (outputs hold NaN)";
    case MOE_E_RANGE: return "a decode-stack value outside the fixed-point range (outputs hold NaN)";
    case MOE_E_OVERLAP: return "an output buffer overlaps an input buffer";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(int64_t T, int32_t D, int32_t F, int32_t E, int32_t k, int32_t format,
                           int32_t flags) {
  (void)format;
  if (T <= 0 || D <= 0 || F <= 0 || E <= 0 || k <= 0) return 0;
  return carve_workspace(nullptr, T, D, F, E, k, flags).bytes;
}

moe_status moe_route(const float* x, int64_t T, int32_t D, const float* gate, const float* bias,
                     int32_t E, int32_t k, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(T, D, E, k));
  if (T == 0) return MOE_OK;
  if (!x || !gate || !topk_ids || !topk_w) return MOE_E_NULLPTR;
  if (!aligned(x, 4) || !aligned(gate, 4) || (bias && !aligned(bias, 4)) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return MOE_E_ALIGN;
  const size_t need = moe_workspace_bytes(T, D, QK, E, k, 0, 0);
  if (!ws || ws_bytes < need) return MOE_E_WORKSPACE;
  const Workspace w = carve_workspace(ws, T, D, QK, E, k, 0);
  trace("route", T, D, 0, E, k, -1);
  return do_route(x, T, D, gate, bias, E, k, topk_ids, topk_w, w, (hipStream_t)stream);
}

moe_status moe_group(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                     int32_t* expert_offsets, int32_t* sorted_rows, void* ws, size_t ws_bytes,
                     void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (T < 0 || E <= 0 || k <= 0 || k > E) return MOE_E_SHAPE;
  if (E > MAX_E || k > MAX_K) return MOE_E_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !expert_offsets || !sorted_rows) return MOE_E_NULLPTR;
  if (!aligned(topk_ids, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_rows, 4))
    return MOE_E_ALIGN;
  trace("group", T, 0, 0, E, k, -1);
  if (launch_group(topk_ids, T * k, E, expert_offsets, sorted_rows, (hipStream_t)stream) !=
      hipSuccess)
    return MOE_E_HIP;
  return MOE_OK;
}

moe_status moe_expert_ffn(const float* in, int32_t stage, const moe_experts* W,
                          const int32_t* topk_ids, const float* topk_w,
                          const int32_t* expert_offsets, const int32_t* sorted_rows, int64_t T,
                          int32_t k, float* y, float* out, int32_t flags, void* ws,
                          size_t ws_bytes, void* stream) {
  MOE_TRY(check_experts(W));
  if (stage != MOE_STAGE_FULL && stage != MOE_STAGE_DOWN) return MOE_E_FORMAT;
  MOE_TRY(check_dims(T, W->d_model, W->num_experts, k));
  if (T == 0) return MOE_OK;
  if (stage == MOE_STAGE_FULL) MOE_TRY(check_gate_up(W));
  if (!in || !topk_ids || !expert_offsets || !sorted_rows) return MOE_E_NULLPTR;
  if (!y && !out) return MOE_E_NULLPTR;
  if (out && !topk_w) return MOE_E_NULLPTR;
  if (!aligned(in, 4) || !aligned(topk_ids, 4) || (topk_w && !aligned(topk_w, 4)) ||
      (y && !aligned(y, 4)) || (out && !aligned(out, 4)) || !aligned(expert_offsets, 4) ||
      !aligned(sorted_rows, 4))
    return MOE_E_ALIGN;
  const size_t need =
      moe_workspace_bytes(T, W->d_model, W->d_ff, W->num_experts, k, W->format, flags);
  if (!ws || ws_bytes < need) return MOE_E_WORKSPACE;
  {
    const size_t rows = (size_t)T * (stage == MOE_STAGE_FULL ? 1 : k);
    const size_t in_b = rows * (stage == MOE_STAGE_FULL ? W->d_model : W->d_ff) * 4;
    if ((out && overlaps(in, in_b, out, (size_t)T * W->d_model * 4)) ||
        (y && overlaps(in, in_b, y, (size_t)T * k * W->d_model * 4)) ||
        (y && out && overlaps(y, (size_t)T * k * W->d_model * 4, out, (size_t)T * W->d_model * 4)))
      return MOE_E_OVERLAP;
  }
  const Workspace w = carve_workspace(ws, T, W->d_model, W->d_ff, W->num_experts, k, flags);
  return do_ffn(in, stage, to_dev(*W), topk_ids, topk_w, expert_offsets, sorted_rows, T, k, y, out,
                flags, w, (hipStream_t)stream);
}

moe_status moe_combine(const float* y, const float* topk_w, int64_t T, int32_t k, int32_t D,
                       const float* residual, float* out, void* stream) {
  if (T < 0 || k <= 0 || D <= 0) return MOE_E_SHAPE;
  if (T == 0) return MOE_OK;
  if (!y || !topk_w || !out) return MOE_E_NULLPTR;
  if (!aligned(y, 4) || !aligned(topk_w, 4) || !aligned(out, 4) ||
      (residual && !aligned(residual, 4)))
    return MOE_E_ALIGN;
  {
    // out may be the residual itself (each element is read before it is written by
    // the same thread), but no other overlap
    const size_t ob = (size_t)T * D * 4;
    if (overlaps(y, (size_t)T * k * D * 4, out, ob) || overlaps(topk_w, (size_t)T * k * 4, out, ob) ||
        (residual && residual != out && overlaps(residual, ob, out, ob)))
      return MOE_E_OVERLAP;
  }
  trace("combine", T, D, 0, 0, k, -1);
  if (launch_combine(y, topk_w, T, k, D, residual, out, (hipStream_t)stream) != hipSuccess)
    return MOE_E_HIP;
  return MOE_OK;
}

moe_status moe_layer(const float* x, const float* gate, const float* bias, const moe_experts* W,
                     int64_t T, int32_t k, int32_t flags, float* out, int32_t* topk_ids,
                     float* topk_w, int32_t* expert_offsets, int32_t* sorted_rows, void* ws,
                     size_t ws_bytes, void* stream) {
  MOE_TRY(check_experts(W));
  MOE_TRY(check_gate_up(W));
  const int D = W->d_model, F = W->d_ff, E = W->num_experts;
  MOE_TRY(check_dims(T, D, E, k));
  if (T == 0) return MOE_OK;
  if (!x || !gate || !out) return MOE_E_NULLPTR;
  if (!aligned(x, 4) || !aligned(gate, 4) || (bias && !aligned(bias, 4)) || !aligned(out, 4) ||
      (topk_ids && !aligned(topk_ids, 4)) || (topk_w && !aligned(topk_w, 4)) ||
      (expert_offsets && !aligned(expert_offsets, 4)) || (sorted_rows && !aligned(sorted_rows, 4)))
    return MOE_E_ALIGN;
  const size_t need = moe_workspace_bytes(T, D, F, E, k, W->format, flags);
  if (!ws || ws_bytes < need) return MOE_E_WORKSPACE;
  if (overlaps(x, (size_t)T * D * 4, out, (size_t)T * D * 4)) return MOE_E_OVERLAP;
  return layer_impl(x, gate, bias, W, T, k, flags, out, topk_ids, topk_w, expert_offsets,
                    sorted_rows, ws, (hipStream_t)stream);
}

moe_status moe_layer_noalloc(const float* x, const float* gate, const float* bias,
                             const moe_experts* W, int64_t T, int32_t k, int32_t flags, float* out,
                             int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                             int32_t* sorted_rows, void* stream) {
  MOE_TRY(check_experts(W));
  MOE_TRY(check_gate_up(W));
  const int D = W->d_model, F = W->d_ff, E = W->num_experts;
  MOE_TRY(check_dims(T, D, E, k));
  if (T == 0) return MOE_OK;
  if (!x || !gate || !out) return MOE_E_NULLPTR;
  if (!aligned(x, 4) || !aligned(gate, 4) || (bias && !aligned(bias, 4)) || !aligned(out, 4) ||
      (topk_ids && !aligned(topk_ids, 4)) || (topk_w && !aligned(topk_w, 4)) ||
      (expert_offsets && !aligned(expert_offsets, 4)) || (sorted_rows && !aligned(sorted_rows, 4)))
    return MOE_E_ALIGN;
  if (moe_workspace_bytes(T, D, F, E, k, W->format, flags) > NOALLOC_SCRATCH_BYTES) {
    if (trace_enabled())
      fprintf(stderr, "[moe] moe_layer_noalloc: T=%lld needs more than the %zu-byte scratch\n",
              (long long)T, NOALLOC_SCRATCH_BYTES);
    return MOE_E_UNSUPPORTED;
  }
  if (overlaps(x, (size_t)T * D * 4, out, (size_t)T * D * 4)) return MOE_E_OVERLAP;
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  MOE_TRY(scratch_for_device(s, &ws));
  return layer_impl(x, gate, bias, W, T, k, flags, out, topk_ids, topk_w, expert_offsets,
                    sorted_rows, ws, s);
}

moe_status moe_decode_stack(const float* x, int32_t num_layers, const moe_stack_layer* layers,
                            int32_t k, int32_t flags, float* outs, int32_t* topk_ids,
                            float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  if (num_layers <= 0) return MOE_E_SHAPE;
  if (!layers || !x || !outs) return MOE_E_NULLPTR;
  if (flags & ~(MOE_F_PRENORM | MOE_F_RESIDUAL | MOE_F_DETERMINISTIC)) return MOE_E_FORMAT;
  const moe_experts* W0 = &layers[0].experts;
  for (int l = 0; l < num_layers; ++l) {
    const moe_experts* W = &layers[l].experts;
    MOE_TRY(check_experts(W));
    MOE_TRY(check_gate_up(W));
    if (W->d_model != W0->d_model || W->d_ff != W0->d_ff || W->num_experts != W0->num_experts)
      return MOE_E_SHAPE;
    if (!layers[l].gate) return MOE_E_NULLPTR;
    if (!aligned(layers[l].gate, 4) || (layers[l].bias && !aligned(layers[l].bias, 4)))
      return MOE_E_ALIGN;
  }
  const int D = W0->d_model, F = W0->d_ff, E = W0->num_experts;
  MOE_TRY(check_dims(1, D, E, k));
  if (!aligned(x, 4) || !aligned(outs, 4) || (topk_ids && !aligned(topk_ids, 4)) ||
      (topk_w && !aligned(topk_w, 4)))
    return MOE_E_ALIGN;
  size_t need = 0;
  for (int l = 0; l < num_layers; ++l) {
    const size_t n = moe_workspace_bytes(1, D, F, E, k, layers[l].experts.format,
                                         MOE_F_PRENORM | MOE_F_RESIDUAL);
    need = n > need ? n : need;
  }
  if (!ws || ws_bytes < need) return MOE_E_WORKSPACE;
  if (overlaps(x, (size_t)D * 4, outs, (size_t)num_layers * D * 4)) return MOE_E_OVERLAP;
  hipStream_t s = (hipStream_t)stream;
  const Workspace w = carve_workspace(ws, 1, D, F, E, k, MOE_F_PRENORM | MOE_F_RESIDUAL);

  bool fused = decode_stack_io_ok(x, outs);
  for (int l = 0; l < num_layers && fused; ++l) {
    const ExpertsDev dv = to_dev(layers[l].experts);
    fused = decode_stack_layer_ok(dv, k) && dv.fmt == W0->format;
  }
  const int LM = decode_stack_max_layers();
  if (fused) {
    trace("decode stack fused", 1, D, F, E, k, W0->format);
    StackLayer sl[64];
    for (int c = 0; c < num_layers; c += LM) {
      const int n = num_layers - c < LM ? num_layers - c : LM;
      for (int i = 0; i < n; ++i)
        sl[i] = StackLayer{layers[c + i].gate, layers[c + i].bias, to_dev(layers[c + i].experts)};
      const float* in = c == 0 ? x : outs + (size_t)(c - 1) * D;
      const bool pre = c > 0 || (flags & MOE_F_PRENORM);
      HIP_TRY(launch_decode_stack(in, n, sl, W0->format, pre, true, outs + (size_t)c * D,
                                  topk_ids ? topk_ids + (size_t)c * k : nullptr,
                                  topk_w ? topk_w + (size_t)c * k : nullptr, nullptr, nullptr,
                                  w, s));
    }
    return MOE_OK;
  }
  trace("decode stack per layer", 1, D, F, E, k, W0->format);
  for (int l = 0; l < num_layers; ++l) {
    const float* in = l == 0 ? x : outs + (size_t)(l - 1) * D;
    const int fl = MOE_F_RESIDUAL | MOE_F_DETERMINISTIC |
                   ((l > 0 || (flags & MOE_F_PRENORM)) ? MOE_F_PRENORM : 0);
    MOE_TRY(layer_impl(in, layers[l].gate, layers[l].bias, &layers[l].experts, 1, k, fl,
                       outs + (size_t)l * D, topk_ids ? topk_ids + (size_t)l * k : nullptr,
                       topk_w ? topk_w + (size_t)l * k : nullptr, nullptr, nullptr, ws, s));
  }
  return MOE_OK;
}

moe_status moe_workspace_status(void* ws, size_t ws_bytes, int32_t reset, void* stream) {
  if (!ws) return MOE_E_NULLPTR;
  if (ws_bytes < ERR_WORD_OFF + sizeof(uint32_t)) return MOE_E_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  uint32_t word = 0;
  char* base = (char*)ws;
  if (hipMemcpyAsync(&word, base + ERR_WORD_OFF, sizeof(word), hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_E_HIP;
  if (word == 0) return MOE_OK;
  if (reset) {
    // the launch counters may disagree after a timeout: zero the whole exchange region
    const size_t n = ws_bytes < SYNC_BYTES ? ws_bytes : SYNC_BYTES;
    if (hipMemsetAsync(ws, 0, n, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
      return MOE_E_HIP;
  }
  return (word & 1u) ? MOE_E_TIMEOUT : MOE_E_RANGE;
}

size_t moe_attn_workspace_bytes(int64_t T, const moe_attn_weights* W) {
  if (T <= 0 || !W || W->n_q_heads <= 0 || W->n_kv_heads <= 0 || W->head_dim <= 0) return 0;
  const int N = (W->n_q_heads + 2 * W->n_kv_heads) * W->head_dim;
  return attn_count_offset(T, N) +
         (size_t)((T + 7) / 8) * (size_t)(W->n_q_heads + W->n_kv_heads) * sizeof(uint32_t);
}

moe_status moe_attn_prep(const float* x, int64_t T, const moe_attn_weights* W, const int32_t* pos,
                         float rope_theta, float eps, float* q, float* k_cache, float* v_cache,
                         int32_t max_pos, void* ws, size_t ws_bytes, void* stream) {
  if (!W) return MOE_E_NULLPTR;
  if (W->format != MOE_FMT_Q8_0 && W->format != MOE_FMT_Q4) return MOE_E_FORMAT;
  const int D = W->d_model, Hq = W->n_q_heads, Hkv = W->n_kv_heads, hd = W->head_dim;
  if (T < 0 || D <= 0 || D % QK || Hq <= 0 || Hkv <= 0 || hd <= 0 || hd % 16 || max_pos < 0)
    return MOE_E_SHAPE;
  if (D > 3584 || hd > 256 || Hq > 1024 || Hkv > 1024) return MOE_E_UNSUPPORTED;   // LDS <= 90 KB
  if (!(rope_theta > 1.0f) || !(eps >= 0.0f)) return MOE_E_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !pos || !q || !W->w_qkv || !W->attn_gain || !W->q_gain || !W->k_gain) return MOE_E_NULLPTR;
  if (max_pos > 0 && (!k_cache || !v_cache)) return MOE_E_NULLPTR;
  if (!aligned(x, 16) || !aligned(W->w_qkv, 16) || !aligned(W->attn_gain, 16) ||
      !aligned(W->q_gain, 4) || !aligned(W->k_gain, 4) || !aligned(pos, 4) || !aligned(q, 4) ||
      (k_cache && !aligned(k_cache, 4)) || (v_cache && !aligned(v_cache, 4)))
    return MOE_E_ALIGN;
  const size_t need = moe_attn_workspace_bytes(T, W);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return MOE_E_WORKSPACE;
  {
    const size_t xb = (size_t)T * D * 4, qb = (size_t)T * Hq * hd * 4;
    const size_t cb = (size_t)max_pos * Hkv * hd * 4;
    if (overlaps(x, xb, q, qb) || overlaps(x, xb, k_cache, cb) || overlaps(x, xb, v_cache, cb) ||
        overlaps(q, qb, k_cache, cb) || overlaps(q, qb, v_cache, cb) ||
        overlaps(k_cache, cb, v_cache, cb))
      return MOE_E_OVERLAP;
  }
  trace("attn prep", T, D, hd, Hq, Hkv, W->format);
  if (launch_attn_prep(x, T, D, W->attn_gain, (const uint8_t*)W->w_qkv, W->format, Hq, Hkv, hd,
                       W->q_gain, W->k_gain, pos, rope_theta, eps, q, k_cache, v_cache, max_pos,
                       ws, (hipStream_t)stream) != hipSuccess)
    return MOE_E_HIP;
  return MOE_OK;
}

moe_status moe_rmsnorm(const float* x, int64_t T, int32_t D, float eps, float* out, void* stream) {
  if (T < 0 || D <= 0) return MOE_E_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !out) return MOE_E_NULLPTR;
  if (!aligned(x, 4) || !aligned(out, 4)) return MOE_E_ALIGN;
  if (!(eps >= 0.0f)) return MOE_E_SHAPE;
  if (launch_rmsnorm(x, T, D, eps, out, (hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

}  // extern "C"
