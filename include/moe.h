/*
 * moe.h -- C ABI of the routed Mixture-of-Experts layer for MI355X (gfx950).
 *
 * The layer is the "router -> resident expert -> combine" segment of MER's warm
 * decode path (technical-overview page, "Execution architecture": warm target
 * path GPU state -> attention -> router -> resident expert -> combine -> next
 * layer; "Next architecture stage": GPU routing, Q4 expert execution, weighted
 * combine).  Geometry it is tuned for: d_model 2048, d_ff 768, 128 experts,
 * top-8 (evidence page, "Historical baseline environment", Model card).  Any
 * d_model / d_ff that is a multiple of 32, 1 <= k <= E <= 1024, k <= 32 runs on
 * the generic kernels.
 *
 * Conventions for every call
 *  - Pointers named in the signature are DEVICE pointers unless the comment
 *    says host.  fp32 arrays are row-major and 4-byte aligned.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  No call except moe_workspace_status (a diagnostic, documented
 *    below) synchronises with the host or copies device -> host, so
 *    data-dependent sizes (per-expert counts) stay on the device and every
 *    call can be captured in a HIP graph.  The hidden state never re-enters
 *    the host between calls (technical-overview page, "Target boundary").
 *  - Ownership: the caller owns every buffer, including the workspace `ws`
 *    (size from moe_workspace_bytes).  The library allocates no device memory
 *    and keeps no mutable state between calls other than inside `ws`: the
 *    first 4 MiB of a workspace hold the launch counters and tagged exchange
 *    words of the fused kernels (single-token decode, decode stack, small-batch
 *    routing), so a workspace must be zero-filled once before its first use
 *    and must not be shared by calls that may run concurrently (calls that
 *    share a workspace must be stream-ordered).
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    on an error the call returns a status != MOE_OK and enqueues nothing.
 *    MOE_E_HIP means a launch failed.  T == 0 is valid and enqueues nothing.
 *  - Device-side errors: the fused kernels (single-token decode, decode stack,
 *    small-batch routing) hand data between workgroups through tagged words
 *    and need all their workgroups resident at once.  Every wait is bounded
 *    (about a second of polling per launch); a wait that gives up sets the
 *    u32 error word at byte 64 of the workspace to nonzero and returns NaN to
 *    the code waiting on it, so the outputs that depend on it are NaN, never
 *    stale data, and every launch still ends.  Causes: other work holding
 *    compute units while a fused kernel runs, or a workspace that was not
 *    zero-filled before first use.  Since the calls never synchronise, the
 *    word is read with moe_workspace_status, which waits for the stream.
 *  - Data preconditions checked on the device rather than the host: expert ids
 *    outside [0, E) are dropped (the affected row contributes nothing to out,
 *    its row of y is zero, and expert_offsets[E] ends below T*k).
 *
 * Block formats (weights are "native Q8_0", evidence page, GPU-native
 * foundation card; 4-bit experts: "Q4 expert execution", technical-overview
 * page, Execution architecture):
 *  - MOE_FMT_Q8_0: 34-byte blocks: fp16 scale d (little-endian) + 32 int8 q;
 *    weight = d * q.
 *  - MOE_FMT_Q4:   18-byte blocks: fp16 scale d + 16 bytes of nibbles, element
 *    2i in the low nibble of byte i, 2i+1 in the high nibble; weight = d*(q-8).
 *  A weight matrix with logical shape [in][out] is stored as `out` rows of
 *  in/32 consecutive blocks (row n = output column n): gate and up are F rows
 *  of D/32 blocks, down is D rows of F/32 blocks.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_E_NULLPTR = 1,     /* a required pointer is NULL                          */
  MOE_E_SHAPE = 2,       /* T < 0, D or F not a positive multiple of 32, bad k/E */
  MOE_E_ALIGN = 3,       /* misaligned pointer or stride                         */
  MOE_E_FORMAT = 4,      /* unknown block format or stage                        */
  MOE_E_WORKSPACE = 5,   /* ws NULL or smaller than moe_workspace_bytes          */
  MOE_E_UNSUPPORTED = 6, /* limits: E > 1024, k > 32, D or F > 16384              */
  MOE_E_HIP = 7,         /* a HIP launch failed                                   */
  MOE_E_TIMEOUT = 8,     /* moe_workspace_status: a fused kernel's bounded wait   */
                         /* gave up since the word was last cleared               */
  MOE_E_RANGE = 9,       /* moe_workspace_status: a fused decode stack met a value */
                         /* outside its fixed-point range (outputs hold NaN)      */
  MOE_E_OVERLAP = 10     /* an output buffer overlaps an input buffer            */
};

enum { MOE_FMT_Q8_0 = 0, MOE_FMT_Q4 = 1 };

/* Stage of moe_expert_ffn. */
enum {
  MOE_STAGE_FULL = 0, /* in = x [T][D]: gate/up -> SwiGLU -> down                 */
  MOE_STAGE_DOWN = 1  /* in = h [T*k][F] in flat (t, j) order: down only          */
};

/* Flags. */
enum {
  MOE_F_RESIDUAL = 1,      /* out += layer input                                       */
  MOE_F_DETERMINISTIC = 2, /* accepted, no effect: every path's fp outputs are already */
                           /* bit-reproducible run to run (ordered sums, exact       */
                           /* fixed-point accumulators)                              */
  MOE_F_PRENORM = 4,       /* moe_layer only: the layer input is rmsnorm(x, eps=1e-6)   */
  MOE_F_FP16_ACT = 8,      /* MFMA expert kernels: round activations to fp16 once       */
                           /* instead of carrying them as two fp16 terms (hi + lo); half */
                           /* the matrix work, ~1e-3 RMS-relative output error           */
  MOE_F_BANDED = 16        /* MFMA down projection: walk the output tiles in bands of   */
                           /* four (reuse-ordering page, "What changed from the first    */
                           /* experiment"); same per-tile arithmetic, so bit-identical   */
                           /* results; off by default (no measured gain on MI355X)       */
};

/* One layer's experts (host struct holding device pointers).  Expert e's gate
 * matrix starts at w_gate + e*gate_stride bytes, likewise up and down.  Bases
 * and strides must be even (fp16 scales); the tuned kernels want 16-byte
 * aligned bases, strides and row sizes and fall back to generic kernels
 * otherwise. */
typedef struct {
  int32_t num_experts; /* E */
  int32_t d_model;     /* D */
  int32_t d_ff;        /* F */
  int32_t format;      /* MOE_FMT_* */
  const void* w_gate;
  int64_t gate_stride;
  const void* w_up;
  int64_t up_stride;
  const void* w_down;
  int64_t down_stride;
} moe_experts;

/* Bytes of device workspace the calls below need for this shape (the maximum
 * over moe_route, moe_group, moe_expert_ffn and moe_layer).  Pure host
 * arithmetic; 0 for T == 0. */
size_t moe_workspace_bytes(int64_t T, int32_t D, int32_t F, int32_t E, int32_t k,
                           int32_t format, int32_t flags);

/* LinearGate router (evidence page, "Layer-qualified experts" card: real
 * LinearGate selection; top-8 in the Model card).
 *   logits l = x G + bias, x [T][D], G [D][E] row-major, bias [E] or NULL.
 *   topk_ids [T][k] int32: the k experts with the largest logits, ties to the
 *     lower expert index, written in ascending id order.
 *   topk_w [T][k] fp32: softmax over all E logits, renormalised over the
 *     selected k (equal to the softmax of the selected logits); sums to 1.
 * Logits are accumulated in fp32.  A -inf logit (an expert masked by a -inf
 * bias) ranks below every finite one and gets weight 0 when fewer than k are
 * finite (ties among -inf go to the lower index).  NaN logits give
 * unspecified ids, always within [0, E). */
moe_status moe_route(const float* x, int64_t T, int32_t D, const float* gate, const float* bias,
                     int32_t E, int32_t k, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, void* stream);

/* Compact per-expert grouping (the reuse-ordering page's "existing compact
 * expert grouping", section "What changed from the first experiment").
 *   expert_offsets [E+1] int32: exclusive scan of per-expert counts,
 *     expert_offsets[E] = number of valid entries (T*k).
 *   sorted_rows [T*k] int32: flat indices t*k + j grouped by expert ascending,
 *     ascending inside each expert (a stable sort by expert id).
 * Integer only; identical on every run. */
moe_status moe_group(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                     int32_t* expert_offsets, int32_t* sorted_rows, void* ws, size_t ws_bytes,
                     void* stream);

/* Routed expert SwiGLU FFNs.
 * Precision: products of exactly decoded weights and activations accumulate in
 * fp32.  When D and F are multiples of 128 (and weight bases / strides are
 * 8-byte aligned, fp32 buffers 16-byte aligned) the grouped MFMA kernels run:
 * activations enter the matrix cores as two fp16 terms (hi + lo, about fp32
 * accuracy), or as one fp16 rounding with MOE_F_FP16_ACT; |activations| must
 * stay below 65504.  Other shapes take generic fp32 kernels.
 * Combine: the grouped kernels store y and the weighted sum runs over it in j
 * order (bit-reproducible); the generic kernels do the same.
 *   stage MOE_STAGE_FULL: in = x [T][D]; for row r = t*k + j with e = ids[t][j]:
 *     h = silu(x_t W_gate_e) * (x_t W_up_e), y_r = h W_down_e.
 *   stage MOE_STAGE_DOWN: in = h [T*k][F]; y_r = h_r W_down_e (the routed
 *     down-projection operator of the reuse-ordering page, K = 768,
 *     2,048 output rows, 128 experts, top-8).
 *   y   [T*k][D] fp32 flat (t, j) order, or NULL;
 *   out [T][D] fp32 = sum_j topk_w[t][j] y_{t*k+j} (+ x_t with MOE_F_RESIDUAL,
 *     stage FULL only), or NULL.  At least one of y / out is non-NULL.
 *   expert_offsets / sorted_rows come from moe_group on the same ids.
 *   y and out must not overlap `in` or each other (MOE_E_OVERLAP, checked on
 *   the host before anything is enqueued). */
moe_status moe_expert_ffn(const float* in, int32_t stage, const moe_experts* W /* host */,
                          const int32_t* topk_ids, const float* topk_w,
                          const int32_t* expert_offsets, const int32_t* sorted_rows, int64_t T,
                          int32_t k, float* y, float* out, int32_t flags, void* ws,
                          size_t ws_bytes, void* stream);

/* Weighted combine (technical-overview page: "weighted combine").
 *   out[t] = sum_{j<k} topk_w[t][j] * y[t*k+j] (+ residual[t] when non-NULL),
 *   summed in j order.  y [T*k][D], out [T][D].  out may be residual itself
 *   (in place); any other overlap of out with an input is MOE_E_OVERLAP. */
moe_status moe_combine(const float* y, const float* topk_w, int64_t T, int32_t k, int32_t D,
                       const float* residual, float* out, void* stream);

/* One whole MoE layer: route -> group -> expert FFNs -> combine, enqueued with
 * no host synchronisation (evidence page: fewer warm host synchronisations;
 * no intermediate host re-entry).
 *   x [T][D]; gate [D][E]; bias [E] or NULL; out [T][D].
 *   With MOE_F_PRENORM the layer input is u = x / sqrt(mean(x^2) + 1e-6)
 *   (the RMSNorm transition between stacked layers), else u = x; with
 *   MOE_F_RESIDUAL out = u + MoE(u), else out = MoE(u).
 *   topk_ids, topk_w, expert_offsets, sorted_rows: optional outputs (NULL =
 *   kept in the workspace only).
 *   out must not overlap x: workgroups still reading x could see outputs
 *   (MOE_E_OVERLAP, checked on the host before anything is enqueued).
 * One token at the tuned geometry (D 2048, F 768, E 128, k 8, 16-byte aligned
 * weight bases and strides, x and out) runs as one launch of the decode-stack
 * kernel (see moe_decode_stack: bit-reproducible, fixed-point sums, the same
 * range limits, reported by moe_workspace_status). */
moe_status moe_layer(const float* x, const float* gate, const float* bias,
                     const moe_experts* W /* host */, int64_t T, int32_t k, int32_t flags,
                     float* out, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                     int32_t* sorted_rows, void* ws, size_t ws_bytes, void* stream);

/* moe_layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and kernels as moe_layer, with the workspace replaced by a static
 * 8 MiB device array inside the library (one per GPU, held until the process
 * ends).  The call allocates nothing and calls no allocating routine; the
 * caller still passes inputs and outputs, as for moe_layer.
 *  - Limit: moe_workspace_bytes(T, D, F, E, k, format, flags) must be at most
 *    8 MiB (8,388,608 bytes): at d_model 2048, d_ff 768, 128 experts, top-8
 *    that is T <= 34 tokens with MOE_F_PRENORM, T <= 36 without.  Larger calls
 *    return MOE_E_UNSUPPORTED and enqueue nothing.
 *  - Every call on a GPU shares that GPU's array, which keeps the last call's
 *    contents: calls that may overlap on one GPU (concurrent streams, several
 *    host threads) race and must be ordered by the caller.
 *  - The first call on a device enqueues a zero fill of the array's exchange
 *    region ahead of its own work on `stream`.
 *  - A fused kernel's exchange wait that gives up makes the outputs NaN, as in
 *    moe_layer; the error word sits in the library's array and is not readable
 *    through moe_workspace_status. */
moe_status moe_layer_noalloc(const float* x, const float* gate, const float* bias,
                             const moe_experts* W /* host */, int64_t T, int32_t k, int32_t flags,
                             float* out, int32_t* topk_ids, float* topk_w,
                             int32_t* expert_offsets, int32_t* sorted_rows, void* stream);

/* One layer of a decode stack (host struct holding device pointers). */
typedef struct {
  const float* gate;   /* [D][E] fp32 LinearGate matrix */
  const float* bias;   /* [E] fp32 logit bias, or NULL */
  moe_experts experts; /* the layer's experts */
} moe_stack_layer;

/* Single-token decode through num_layers consecutive MoE layers, each with its
 * residual add, and the RMSNorm transition between layers (evidence page:
 * "RMSNorm and residual transitions"; technical-overview page, warm target
 * path ... router -> resident expert -> combine -> next layer):
 *   in_0 = x, or x / sqrt(mean(x^2) + 1e-6) with MOE_F_PRENORM (for a stack
 *   that continues an earlier one, x being its last output);
 *   o_l = in_l + MoE_l(in_l);  in_{l+1} = o_l / sqrt(mean(o_l^2) + 1e-6).
 * The whole stack is enqueued with no host synchronisation; on the tuned
 * geometry (D 2048, F 768, E 128, k 8, every layer in one format, 16-byte
 * aligned weight bases and strides) one persistent launch runs up to 24
 * layers with no launch between them, and its fp outputs are
 * bit-reproducible: each layer's output o_l and the next router's logits are
 * summed across workgroups in 64-bit fixed point (2^-24 resolution, exact and
 * independent of arrival order).  There a contribution to o_l (a slot's
 * w_j y_j(d), or the residual) must stay below 2^27 in magnitude and a
 * 64-row partial logit below 2^13; beyond that the outputs from that layer on
 * are NaN and moe_workspace_status reports MOE_E_RANGE.  Other shapes run
 * moe_layer per layer.
 *   x [D] fp32 (one token); layers: host array of num_layers >= 1 entries;
 *   outs [num_layers][D] fp32: o_l of every layer; must not overlap x
 *   (MOE_E_OVERLAP);
 *   topk_ids [num_layers][k] int32, topk_w [num_layers][k] fp32: optional
 *   (NULL) routing of every layer, as moe_route reports it.
 *   flags: MOE_F_PRENORM or 0 (MOE_F_RESIDUAL and MOE_F_DETERMINISTIC are
 *   implied and accepted).  ws: moe_workspace_bytes(1, D, F, E, k, format,
 *   MOE_F_PRENORM) bytes, zero-filled before first use like every workspace. */
moe_status moe_decode_stack(const float* x, int32_t num_layers,
                            const moe_stack_layer* layers /* host */, int32_t k, int32_t flags,
                            float* outs, int32_t* topk_ids, float* topk_w, void* ws,
                            size_t ws_bytes, void* stream);

/* Attention-side weights of one layer (host struct holding device pointers)
 * for moe_attn_prep. */
typedef struct {
  int32_t d_model;          /* D: multiple of 32, at most 3584                          */
  int32_t n_q_heads;        /* Hq >= 1                                                   */
  int32_t n_kv_heads;       /* Hkv >= 1                                                  */
  int32_t head_dim;         /* hd: multiple of 16, at most 256                           */
  int32_t format;           /* MOE_FMT_* of w_qkv                                        */
  const void* w_qkv;        /* (Hq + 2 Hkv) * hd stored rows of D/32 blocks: the q rows
                               of head 0..Hq-1, then the k rows of head 0..Hkv-1, then
                               the v rows (row n = output n); 16-byte aligned           */
  const float* attn_gain;   /* [D] gain of the input RMSNorm; 16-byte aligned            */
  const float* q_gain;      /* [hd] gain of the per-head q RMSNorm                       */
  const float* k_gain;      /* [hd] gain of the per-head k RMSNorm                       */
} moe_attn_weights;

/* Bytes of workspace moe_attn_prep needs: 256 header bytes (the error word
 * at byte 64, as in every workspace; read it with moe_workspace_status), the
 * projected q and k rows of every token as tagged 64-bit words (rounded up to
 * 256 bytes), then ceil(T/8) * (Hq + Hkv) u32 counters; 0 for T == 0 or a NULL
 * W.  The workspace must be 256-byte aligned and zero-filled before its first
 * use; the counters keep running across calls. */
size_t moe_attn_workspace_bytes(int64_t T, const moe_attn_weights* W /* host */);

/* The attention-side primitives of the warm decode path (technical-overview
 * page, "Validated GPU foundation": RMSNorm, grouped per-head Q/K
 * normalization, Q/K/V projections, RoPE, request-local F32 KV append).  For
 * each token t:
 *   u = x_t / sqrt(mean(x_t^2) + eps) * attn_gain;
 *   [q | k | v] = u W_qkv (block-quantized rows, fp32 accumulation);
 *   every q head: q_h / sqrt(mean(q_h^2) + eps) * q_gain, every k head likewise
 *   with k_gain (one shared gain per kind, the grouped per-head norm);
 *   RoPE on q and k: for i < hd/2 the pair (e_i, e_{i+hd/2}) is rotated by the
 *   angle pos[t] * rope_theta^(-2i/hd);
 *   q [T][Hq][hd] gets the rotated q; k_cache and v_cache ([max_pos][Hkv][hd]
 *   fp32, caller-owned) get the rotated k and the projected v at row pos[t].
 *   A token whose pos is outside [0, max_pos) writes q only.
 *   x, q, k_cache and v_cache must not overlap (MOE_E_OVERLAP).
 * Causal attention itself (scores, softmax, value aggregation, output
 * projection) is not part of this call.  x [T][D] 16-byte aligned; pos [T]
 * int32; ws at least moe_attn_workspace_bytes, zero-filled before first use,
 * not shared by calls that may overlap.  Asynchronous on `stream`; one launch;
 * results are bit-reproducible. */
moe_status moe_attn_prep(const float* x, int64_t T, const moe_attn_weights* W /* host */,
                         const int32_t* pos, float rope_theta, float eps, float* q,
                         float* k_cache, float* v_cache, int32_t max_pos, void* ws,
                         size_t ws_bytes, void* stream);

/* RMSNorm with unit gain (evidence page: "RMSNorm and residual transitions"):
 * out[t] = x[t] / sqrt(mean_D(x[t]^2) + eps).  out may equal x. */
moe_status moe_rmsnorm(const float* x, int64_t T, int32_t D, float eps, float* out, void* stream);

/* Device-side error word of a workspace (see "Device-side errors" above).
 * SYNCHRONOUS: waits for every call enqueued on `stream` so far, then reads
 * the u32 word at byte 64 of ws (a device pointer).  Returns MOE_OK if it is
 * zero, MOE_E_TIMEOUT if a bounded wait of any call on this workspace gave up
 * since it was last cleared (the outputs of that call hold NaN), otherwise
 * MOE_E_RANGE if a decode stack met a value outside its fixed-point range
 * (see moe_decode_stack; its later outputs hold NaN), MOE_E_HIP if the copy
 * failed, MOE_E_NULLPTR / MOE_E_WORKSPACE for a missing or too small
 * workspace (ws_bytes < 68).  With reset != 0 and an error recorded, the
 * exchange region (the first 4 MiB: launch counters, exchange words and the
 * decode stack's accumulators) is zero-filled before returning, so the
 * workspace is usable again.  Not for graph capture. */
moe_status moe_workspace_status(void* ws, size_t ws_bytes, int32_t reset, void* stream);

/* Host-side helpers. */
const char* moe_status_str(moe_status s);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
