#!/usr/bin/env python3
"""Throughput of the routed MoE layer on one MI355X.

Headline workload (the JSON line's ``value``): single-token decode through
Qwen3-MoE-geometry MoE layers (d_model 2048, d_ff 768, 128 Q8_0 experts,
Zipf-biased LinearGate, top-8).  One step = one token through 48 distinct layers
chained with residual + RMSNorm: one moe_decode_stack call (two persistent
launches of 24 layers), captured once as a HIP graph and replayed.  Consecutive
layers never reuse expert weights, so the 256 MB Infinity Cache cannot serve
them.  ``value`` = routed MoE-layer tokens/s = 48 * steps / elapsed.

The same run also measures, under ``workloads``:
  toy            16 tokens through the toy layer (d_model 256, 16 Q8_0 experts, top-2)
  decode_per_layer  the same 48-layer decode step as 48 moe_layer calls (one fused
                 launch per layer)
  decode_batch   32 tokens x 16 chained 4-bit layers (residual + RMSNorm)
  prefill_down   the down projection operator: 1024 tokens routed top-8 (8192 rows
                 of 768 fp32 activations), 4-bit W_down, rotating over 16 layers'
                 routings and weights; one call = grouping + expert kernels +
                 weighted combine (the grouping is timed with the operator, as the
                 reuse-ordering page timed routing with it); both the two-term
                 (hi+lo fp16) and the single-fp16 activation variants
  prefill_stack  2048 tokens as two 1024-token microbatches through 48 Q8_0
                 layers (residual + RMSNorm), 96 layer calls per pass
  attn_prep      one decode token through the attention-side primitives (input
                 RMSNorm, Q8_0 Q/K/V projection 2048 -> 32+4+4 heads of 128,
                 per-head Q/K RMSNorm, RoPE, KV append), rotating over 48 layers
Each reports its time per call, algorithmic GB/s against the 8 TB/s HBM peak and
algorithmic MFMA TFLOP/s against the 2.5166 PFLOP/s dense fp16 peak (flops
counted once: 2 x rows x K x N per product; the second activation term of the
split mode is not counted).  Algorithmic bytes = expert weights of the U experts
that received rows + router matrix + activations in + outputs out.  Each workload
also carries its own ``cpu_baseline``: the fp64 oracle timed on the host on a
bounded sample of the same workload.

Prints ONE JSON line.  ``roofline`` reports the dominant kernel of the headline
workload (decode_stack_kernel); ``cpu_baseline`` times the fp64 CPU oracle on a
bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2516.6          # 256 CU x 4096 flop/clk x 2.4 GHz, dense
D, F, E, K = 2048, 768, 128, 8
Q8_BLOB = 5_013_504                      # one Q8_0 expert: 3 * 2048 * 768 / 32 * 34 bytes
Q4_BLOB = 2_654_208                      # one 4-bit expert: 3 * 2048 * 768 / 32 * 18 bytes
Q4_DOWN = 884_736                        # one 4-bit W_down: 2048 * 768 / 32 * 18 bytes
GATE_BYTES = D * E * 4 + E * 4           # router matrix + bias
DECODE_ALGO_BYTES = K * Q8_BLOB + GATE_BYTES + 2 * D * 4   # = 41,173,504
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mixture_experts_routed_lineargate_amd", "csrc")
STACK_SRCS = (os.path.join(CSRC, "decode_stack.hip"), os.path.join(CSRC, "decode_common.hpp"))
DOWN_OP_SRCS = tuple(os.path.join(CSRC, f) for f in ("grouped_gemm.hip", "mfma_frag.hpp",
                                                     "ffn_generic.hip", "group.hip"))
PREFILL_SRCS = DOWN_OP_SRCS + (os.path.join(CSRC, "router.hip"),)
BATCH_SRCS = tuple(os.path.join(CSRC, f) for f in ("skinny_gemm.hip", "route_small.hip",
                                                   "mfma_frag.hpp", "ffn_generic.hip"))
ATTN_SRCS = (os.path.join(CSRC, "attn_prep.hip"), os.path.join(CSRC, "decode_common.hpp"))
STACK_LAYERS_PER_LAUNCH = 24
WORKLOADS = ("toy", "decode_per_layer", "decode_batch", "prefill_down", "prefill_stack", "attn_prep")
CPU_BUDGET = {"toy": 2.0, "decode_batch": 6.0, "prefill_down": 6.0, "prefill_stack": 15.0,
              "attn_prep": 3.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--repeats", type=int, default=10,
                    help="timed repeats per workload (median, p10, p90); 1 for profiler runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time budget of the headline's cpu_baseline")
    ap.add_argument("--workloads", default=",".join(WORKLOADS),
                    help="comma list of extra workloads to measure (empty for none)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters in a profiler run)")
    return ap.parse_args()


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(tag: str, srcs, key: str = "traffic_bytes_per_launch"):
    """HBM bytes from a committed rocprofv3 counter summary (profiles/<tag>_traffic.md),
    if it was taken on the current kernel source (its ``source_sha256:`` line)."""
    p = os.path.join(PROFILE_DIR, f"{tag}_traffic.md")
    if not os.path.exists(p):
        return None
    fields = {}
    with open(p) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != source_sha(srcs):
        return None
    try:
        return int(fields[key])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# Oracle timing on the host
# ---------------------------------------------------------------------------

def host_threads() -> dict:
    """Host cores this process may run on, and the BLAS threads numpy uses."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = None
    return {"cores": blas if blas else 1, "host_cores": cores, "blas_threads": blas}


def oracle_rate(run_one, budget_s: float, max_n: int, per_call: float, unit: str, sample: str):
    """Time run_one(i) (the timed part only, as returned) until budget_s is spent."""
    total, n = 0.0, 0
    while total < budget_s and n < max_n:
        total += run_one(n)
        n += 1
    r = {"value": round(n * per_call / total, 4), "unit": unit, "kind": "oracle",
         "sample": sample.format(n=n, s=total)}
    r.update(host_threads())
    return r


def host_experts(arena_l, ids, fmt, Dm=D, Fm=F, which=None):
    import moe_synth as S
    from oracle import moe_oracle as O
    host = {}
    for e in sorted(set(int(e) for e in ids)):
        g, u, d = S.split_blob(arena_l[e].cpu().numpy(), Dm, Fm, fmt)
        host[e] = (g, u, d) if which is None else tuple(m if n in which else None
                                                        for n, m in zip(("gate", "up", "down"),
                                                                        (g, u, d)))
    return O.Experts(lambda e: host[e], fmt)


def cpu_decode(arena, layers_np, budget_s: float):
    """Headline: single-token Q8_0 layers on distinct layers of the arena.  The oracle
    routes first (untimed) so that only the 8 selected experts are copied to the host;
    the timed call is the whole oracle layer (routing, dequantising the 8 experts,
    SwiGLU FFNs, combine)."""
    import moe_synth as S
    from oracle import moe_oracle as O

    def one(n):
        l = (7 * n + 3) % len(layers_np)
        G, b = layers_np[l]
        x = S.hidden(2, 1, D, layer=1000 + n)
        ids = O.select_topk(O.router_logits(x, G, b), K)[0]
        ex = host_experts(arena[l], ids, S.FMT_Q8_0)
        t0 = time.perf_counter()
        O.moe_layer(x, G, b, ex, K, residual=True)
        return time.perf_counter() - t0
    return oracle_rate(one, budget_s, 2000, 1.0, "tokens/s",
                       "{n} single-token Q8_0 decode layer calls on distinct layers (fp64 numpy "
                       "oracle: routing, dequantising the 8 selected experts, SwiGLU, combine); {s:.1f} s")


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

REPEATS = 10      # timed repeats per workload: median, p10 and p90 are reported


def graph_time_reps(torch, fn, stream, warmup: int, iters: int, reps: int) -> list:
    """Capture fn() once as a HIP graph; time `reps` repeats of `iters` replays each (events
    on `stream`) and return the mean ms per replay of every repeat."""
    with torch.cuda.stream(stream):
        fn()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            start.record(stream)
            for _ in range(iters):
                graph.replay()
            end.record(stream)
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) / iters)
    return out


def graph_time_ms(torch, fn, stream, warmup: int, iters: int) -> float:
    """Capture fn() once as a HIP graph; return the mean ms per replay over `iters` replays."""
    return graph_time_reps(torch, fn, stream, warmup, iters, 1)[0]


def percentile(reps: list, f: float, scale: float = 1.0) -> float:
    """The f-th percentile of per-repeat times divided by `scale` (linear interpolation
    between order statistics)."""
    v = sorted(m / scale for m in reps)
    i = f / 100.0 * (len(v) - 1)
    lo = int(i)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (i - lo)


def median_of(reps: list, scale: float = 1.0) -> float:
    return percentile(reps, 50, scale)


def spread(reps: list, scale: float = 1.0) -> dict:
    """Median, p10 and p90 of per-repeat times (ms, each divided by `scale`)."""
    return {"repeats": len(reps), "ms_p10": round(percentile(reps, 10, scale), 6),
            "ms_median": round(percentile(reps, 50, scale), 6),
            "ms_p90": round(percentile(reps, 90, scale), 6)}


def n_active(torch, ids) -> int:
    return int(torch.unique(ids).numel())


def rates(ms: float, nbytes: float, flops: float) -> dict:
    """Algorithmic rates against the HBM and dense fp16 MFMA peaks."""
    s = ms / 1e3
    gbps = nbytes / s / 1e9
    tf = flops / s / 1e12
    return {"ms_per_call": round(ms, 5), "algorithmic_bytes": int(nbytes),
            "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "mfma_tflops": round(tf, 2), "mfma_frac": round(tf / MFMA_FP16_PEAK_TFLOPS, 4)}


def ffn_flops(rows: int, Dm: int = D, Fm: int = F) -> float:
    return 2.0 * rows * Dm * Fm * 3


def bench_toy(torch, M, S, dev, stream, iters, cpu):
    """16 tokens through the toy layer (d_model 256, d_ff 128, 16 Q8_0 experts, top-2)."""
    from oracle import moe_oracle as O
    T, Dm, Fm, Em, k = 16, 256, 128, 16, 2
    G = S.gate_matrix(1, Dm, Em)
    x = S.hidden(1, T, Dm)
    blobs = S.expert_blobs(1, Em, Dm, Fm, S.FMT_Q8_0)
    ex = M.Experts.from_blobs(torch.from_numpy(blobs).to(dev), Dm, Fm, S.FMT_Q8_0)
    tx, tG = torch.from_numpy(x).to(dev), torch.from_numpy(G).to(dev)
    out = torch.empty((T, Dm), dtype=torch.float32, device=dev)
    ws = M.workspace(T, Dm, Fm, Em, k, S.FMT_Q8_0)

    def one():
        M.moe_layer(tx, tG, None, ex, k, out, ws=ws, stream=stream)
    reps = graph_time_reps(torch, one, stream, 3, max(iters, 50), REPEATS)
    ms = median_of(reps)
    r = {"workload": "toy layer: 16 tokens x d_model 256, 16 Q8_0 experts (256x128 / 128x256), "
                     "top-2, no bias (latency-bound; correctness config)",
         "tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_call": round(ms, 5),
         "spread": spread(reps)}
    if cpu:
        oex = O.Experts(lambda e: S.split_blob(blobs[e], Dm, Fm, S.FMT_Q8_0), S.FMT_Q8_0)

        def run(n):
            t0 = time.perf_counter()
            O.moe_layer(x, G, None, O.Experts(oex.fetch, S.FMT_Q8_0), k)
            return time.perf_counter() - t0
        r["cpu_baseline"] = oracle_rate(run, CPU_BUDGET["toy"], 500, T, "tokens/s",
                                        "{n} calls of the whole 16-token toy layer (fp64 oracle, "
                                        "experts decoded per call); {s:.1f} s")
    return r


def bench_decode_batch(torch, M, S, dev, stream, iters, cpu):
    """32 tokens through 16 chained 4-bit layers (residual + RMSNorm), one graph per pass."""
    from oracle import moe_oracle as O
    T, L4 = 32, 16
    arena = S.device_arena(3, L4, E, D, F, S.FMT_Q4, dev)
    gnp = [(S.gate_matrix(3, D, E, layer=l), S.zipf_bias(3, E, layer=l)) for l in range(L4)]
    gates = [(torch.from_numpy(G).to(dev), torch.from_numpy(b).to(dev)) for G, b in gnp]
    ex = [M.Experts.from_blobs(arena[l], D, F, S.FMT_Q4) for l in range(L4)]
    flags = M.F_RESIDUAL | M.F_PRENORM
    ws = M.workspace(T, D, F, E, K, S.FMT_Q4, flags)
    x0 = S.hidden(3, T, D)
    bufs = [torch.from_numpy(x0).to(dev)] + \
           [torch.empty((T, D), dtype=torch.float32, device=dev) for _ in range(L4)]
    ids = torch.empty((L4, T, K), dtype=torch.int32, device=dev)

    def one():
        for l in range(L4):
            M.moe_layer(bufs[l], gates[l][0], gates[l][1], ex[l], K, bufs[l + 1],
                        flags=flags if l > 0 else M.F_RESIDUAL, topk_ids=ids[l], ws=ws,
                        stream=stream)
    reps = graph_time_reps(torch, one, stream, 3, iters, REPEATS)
    ms = median_of(reps, L4)
    M.check_workspace(ws, stream=stream)
    U = sum(n_active(torch, ids[l]) for l in range(L4)) / L4
    nbytes = U * Q4_BLOB + GATE_BYTES + 2 * T * D * 4
    flops = ffn_flops(T * K) + 2.0 * T * D * E
    r = {"workload": "decode batch: 32 tokens x Qwen3-MoE layer, 4-bit experts, Zipf router, top-8; "
                     "16 distinct layers chained (residual + RMSNorm)",
         "tokens_per_s": round(T / (ms / 1e3), 1), "mean_active_experts": round(U, 2)}
    r.update(rates(ms, nbytes, flops))
    r["spread"] = spread(reps, L4)
    r["traffic"] = counter_traffic("decode_batch_q4_layer", BATCH_SRCS)
    if cpu:
        def run(n):
            l = n % L4
            G, b = gnp[l]
            xl = S.hidden(3, T, D, layer=2000 + n)
            eids = O.select_topk(O.router_logits(xl, G, b), K)
            oex = host_experts(arena[l], eids.ravel(), S.FMT_Q4)
            t0 = time.perf_counter()
            O.moe_layer(xl, G, b, oex, K, residual=True)
            return time.perf_counter() - t0
        r["cpu_baseline"] = oracle_rate(run, CPU_BUDGET["decode_batch"], 200, T, "tokens/s",
                                        "{n} calls of one whole 32-token 4-bit layer (fp64 oracle: "
                                        "routing, dequantising the active experts, SwiGLU, "
                                        "combine); {s:.1f} s")
    del arena
    return r


def bench_prefill_down(torch, M, S, dev, stream, iters, cpu):
    """Grouping + down projection + combine over 8192 routed rows, rotating over 16 layers."""
    from oracle import moe_oracle as O
    T, L4 = 1024, 16
    R = T * K
    arena = S.device_arena(4, L4, E, D, F, S.FMT_Q4, dev, which=("down",))
    ex = [M.Experts.from_blobs(arena[l], D, F, S.FMT_Q4) for l in range(L4)]
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    h = torch.randn((R, F), generator=g, device=dev, dtype=torch.float32)
    xr = torch.randn((T, D), generator=g, device=dev, dtype=torch.float32)
    ws = M.workspace(T, D, F, E, K, S.FMT_Q4)
    ids = torch.empty((L4, T, K), dtype=torch.int32, device=dev)
    w = torch.empty((L4, T, K), dtype=torch.float32, device=dev)
    offs = torch.empty((L4, E + 1), dtype=torch.int32, device=dev)
    rows = torch.empty((L4, R), dtype=torch.int32, device=dev)
    for l in range(L4):       # the operator's input routing (setup, untimed)
        G = torch.from_numpy(S.gate_matrix(4, D, E, layer=l)).to(dev)
        b = torch.from_numpy(S.zipf_bias(4, E, layer=l)).to(dev)
        M.moe_route(xr, G, b, K, ids[l], w[l], ws)
    torch.cuda.synchronize()
    out = torch.empty((T, D), dtype=torch.float32, device=dev)
    U = sum(n_active(torch, ids[l]) for l in range(L4)) / L4
    nbytes = U * Q4_DOWN + R * F * 4 + T * D * 4 + R * 4 * 3 + (E + 1) * 4
    flops = 2.0 * R * F * D
    res = {"workload": "prefill down projection operator: 1024 tokens routed top-8 of 128 "
                       "(8192 rows x 768 fp32), 4-bit W_down 768x2048, Zipf routers; one call = "
                       "grouping + expert kernels + weighted combine; rotating over 16 layers",
           "mean_active_experts": round(U, 2)}
    # split_fp16_banded: the same operator with the output tiles walked in bands of
    # four (the reuse-ordering page's traversal; bit-identical results)
    for name, fl in (("split_fp16", 0), ("fp16", M.F_FP16_ACT), ("split_fp16_banded", M.F_BANDED)):
        def one(fl=fl):
            for l in range(L4):
                M.moe_group(ids[l], E, offs[l], rows[l], ws, stream=stream)
                M.moe_expert_ffn(h, M.STAGE_DOWN, ex[l], ids[l], w[l], offs[l], rows[l],
                                 out=out, flags=fl, ws=ws, stream=stream)
        reps = graph_time_reps(torch, one, stream, 3, iters, REPEATS)
        ms = median_of(reps, L4)
        r = {"tokens_per_s": round(T / (ms / 1e3), 1)}
        r.update(rates(ms, nbytes, flops))
        r["spread"] = spread(reps, L4)
        res[name] = r
    res["traffic"] = counter_traffic("prefill_down_q4_operator", DOWN_OP_SRCS)
    if cpu:
        hs = h[:256 * K].cpu().numpy()

        def run(n):
            l = n % L4
            tid = ids[l, :256].cpu().numpy()
            tw = w[l, :256].cpu().numpy()
            oex = host_experts(arena[l], tid.ravel(), S.FMT_Q4, which=("down",))
            t0 = time.perf_counter()
            O.down_combine(hs, tid, tw, oex)
            return time.perf_counter() - t0
        res["cpu_baseline"] = oracle_rate(run, CPU_BUDGET["prefill_down"], 100, 256, "tokens/s",
                                          "{n} calls of the operator on 256 of the 1024 tokens "
                                          "(2048 routed rows; fp64 oracle: dequantising the "
                                          "active W_down, products, combine); {s:.1f} s")
    del arena
    return res


def bench_prefill_stack(torch, M, S, dev, stream, arena, layers_np, gates, iters, cpu):
    """2048 tokens as 2 x 1024 through 48 Q8_0 layers (residual + RMSNorm)."""
    from oracle import moe_oracle as O
    T, MB = 2048, 1024
    L = arena.shape[0]
    ex = [M.Experts.from_blobs(arena[l], D, F, S.FMT_Q8_0) for l in range(L)]
    flags = M.F_RESIDUAL | M.F_PRENORM
    ws = M.workspace(MB, D, F, E, K, S.FMT_Q8_0, flags)
    x0np = S.hidden(5, T, D)
    x0 = torch.from_numpy(x0np).to(dev)
    outs = torch.empty((L, T, D), dtype=torch.float32, device=dev)
    ids = torch.empty((L, T, K), dtype=torch.int32, device=dev)

    def one():
        for mb in range(T // MB):
            sl = slice(mb * MB, (mb + 1) * MB)
            for l in range(L):
                src = x0[sl] if l == 0 else outs[l - 1, sl]
                M.moe_layer(src, gates[l][0], gates[l][1], ex[l], K, outs[l, sl],
                            flags=flags if l > 0 else M.F_RESIDUAL, topk_ids=ids[l, sl], ws=ws,
                            stream=stream)
    reps = graph_time_reps(torch, one, stream, 2, iters, REPEATS)
    ms = median_of(reps)
    M.check_workspace(ws, stream=stream)
    if not torch.isfinite(outs[L - 1]).all():
        raise RuntimeError("prefill stack: non-finite output")
    Us = [n_active(torch, ids[l, mb * MB:(mb + 1) * MB]) for mb in range(T // MB) for l in range(L)]
    nbytes = sum(Us) * Q8_BLOB + len(Us) * (GATE_BYTES + 2 * MB * D * 4)
    flops = len(Us) * (ffn_flops(MB * K) + 2.0 * MB * D * E)
    r = {"workload": "prefill: 2048 tokens as two 1024-token microbatches through 48 Qwen3-MoE "
                     "layers (128 Q8_0 experts each, Zipf routers, top-8, residual + RMSNorm)",
         "tokens_per_s": round(T / (ms / 1e3), 1),
         "token_layers_per_s": round(T * L / (ms / 1e3), 1),
         "mean_active_experts": round(sum(Us) / len(Us), 2)}
    r.update(rates(ms, nbytes, flops))
    r["ms_per_call"] = round(ms / len(Us), 5)
    r["ms_per_pass"] = round(ms, 4)
    r["spread"] = spread(reps)                      # ms per pass
    r["traffic_per_microbatch_layer"] = counter_traffic("prefill_layer_q8_0", PREFILL_SRCS)
    if cpu:
        # once: a 2-token sample (one from each microbatch) through all 48 layers
        sample = x0np[[5, MB + 5]]

        def layers():
            for l in range(L):
                yield layers_np[l][0], layers_np[l][1], lazy_layer(arena[l])

        t0 = time.perf_counter()
        O.stack(sample, layers(), K)
        dt = time.perf_counter() - t0
        r["cpu_baseline"] = {"value": round(2 * L / dt, 4), "unit": "token-layers/s",
                             "kind": "oracle",
                             "sample": f"2 tokens (one per microbatch) through all 48 layers, once "
                                       f"(fp64 oracle stack: routing, dequantising each selected "
                                       f"expert, SwiGLU, combine, residual, RMSNorm); {dt:.1f} s"}
        r["cpu_baseline"].update(host_threads())
    del outs
    return r


def bench_attn(torch, M, S, dev, stream, iters, cpu):
    """One decode token through the attention-side primitives, 48 distinct layers."""
    from oracle import moe_oracle as O
    Dm, nq, nkv, hd, L = 2048, 32, 4, 128, 48
    N = S.qkv_rows(nq, nkv, hd)
    arena = S.device_qkv_arena(6, L, Dm, nq, nkv, hd, S.FMT_Q8_0, dev)
    gnp = [S.attn_gain(6, Dm, 0), S.attn_gain(6, hd, 1), S.attn_gain(6, hd, 2)]
    ga, gq, gk = (torch.from_numpy(g).to(dev) for g in gnp)
    W = [M.AttnWeights(arena[l], ga, gq, gk, Dm, nq, nkv, hd, S.FMT_Q8_0) for l in range(L)]
    max_pos = 8192
    x = torch.from_numpy(S.hidden(6, 1, Dm)).to(dev)
    pos = torch.tensor([4097], dtype=torch.int32, device=dev)
    q = torch.empty((1, nq, hd), dtype=torch.float32, device=dev)
    kc = torch.zeros((L, max_pos, nkv, hd), dtype=torch.float32, device=dev)
    vc = torch.zeros((L, max_pos, nkv, hd), dtype=torch.float32, device=dev)
    ws = M.attn_workspace(1, W[0])

    def one():
        for l in range(L):
            M.moe_attn_prep(x, W[l], pos, q, kc[l], vc[l], ws=ws, stream=stream)
    reps = graph_time_reps(torch, one, stream, 3, iters, REPEATS)
    ms = median_of(reps, L)
    rb = Dm // 32 * 34
    nbytes = N * rb + Dm * 4 * 2 + 2 * hd * 4 + nq * hd * 4 + 2 * nkv * hd * 4 + 4
    r = {"workload": "attention-side primitives, one decode token: input RMSNorm, Q8_0 Q/K/V "
                     "projection 2048 -> (32 + 4 + 4) x 128, per-head Q/K RMSNorm, RoPE, F32 KV "
                     "append; 48 distinct layers",
         "us_per_call": round(ms * 1e3, 3)}
    r.update(rates(ms, nbytes, 2.0 * Dm * N))
    r["spread"] = spread(reps, L)
    # fp32 vector dots, no matrix cores: the MFMA fields do not apply
    r.pop("mfma_tflops", None)
    r.pop("mfma_frac", None)
    r["traffic"] = counter_traffic("attn_prep_q8_0", ATTN_SRCS)
    if cpu:
        xnp = S.hidden(6, 1, Dm)

        def run(n):
            raw = arena[n % L].cpu().numpy()
            t0 = time.perf_counter()
            O.attn_prep(xnp, raw, S.FMT_Q8_0, gnp[0], gnp[1], gnp[2], [4097], 1e6, nq, nkv, hd)
            return time.perf_counter() - t0
        r["cpu_baseline"] = oracle_rate(run, CPU_BUDGET["attn_prep"], 100, 1, "tokens/s",
                                        "{n} single-token calls of the fp64 oracle (dequantising "
                                        "the 5120 x 2048 Q8_0 projection, norms, RoPE); {s:.1f} s")
    del arena, kc, vc
    return r


def lazy_layer(arena_l):
    """The oracle's Experts over one Q8_0 layer of a device arena, bytes fetched per expert."""
    import moe_synth as S
    from oracle import moe_oracle as O
    return O.Experts(lambda e: S.split_blob(arena_l[e].cpu().numpy(), D, F, S.FMT_Q8_0),
                     S.FMT_Q8_0)


def main():
    a = parse()
    global REPEATS
    REPEATS = max(1, a.repeats)
    if a.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; runs on more than one GPU are "
                                   "not part of it (the sharding plan is documented, not run)"}))
        sys.exit(2)
    import torch

    import moe_synth as S
    import mixture_experts_routed_lineargate_amd as M

    dev = torch.device("cuda:0")
    L = a.layers
    cpu = not a.no_cpu_baseline
    arena = S.device_arena(2, L, E, D, F, S.FMT_Q8_0, dev)          # [L][E][stride]
    layers_np = [(S.gate_matrix(2, D, E, layer=l), S.zipf_bias(2, E, layer=l)) for l in range(L)]
    gates = [(torch.from_numpy(G).to(dev), torch.from_numpy(b).to(dev)) for G, b in layers_np]
    experts = [M.Experts.from_blobs(arena[l], D, F, S.FMT_Q8_0) for l in range(L)]
    flags = M.F_RESIDUAL | M.F_PRENORM
    ws = M.workspace(1, D, F, E, K, S.FMT_Q8_0, flags)
    x0 = torch.from_numpy(S.hidden(2, 1, D)).to(dev)
    stream = torch.cuda.Stream()
    want = [w for w in a.workloads.split(",") if w]
    if a.calib_copy_mib:
        n = a.calib_copy_mib << 18                    # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # headline: one moe_decode_stack call per step
    stack_layers = M.StackLayers([g for g, _ in gates], [b for _, b in gates], experts)
    outs = torch.empty((L, D), dtype=torch.float32, device=dev)

    def one_stack():
        M.moe_decode_stack(x0[0], stack_layers, K, outs, ws=ws, stream=stream)

    ms_step = graph_time_ms(torch, one_stack, stream, a.warmup, a.steps)
    # spread: REPEATS further timed runs of steps/10 steps each, after the timed region
    step_reps = graph_time_reps(torch, one_stack, stream, 0, max(1, a.steps // 10), REPEATS)
    M.check_workspace(ws, stream=stream)             # raises if an exchange wait gave up
    if not torch.isfinite(outs).all():
        raise RuntimeError("non-finite output")
    print(f"[bench] decode stack: {ms_step * 1e3 / L:.2f} us per layer", file=sys.stderr, flush=True)

    launches = -(-L // STACK_LAYERS_PER_LAUNCH)
    launch_s = ms_step / 1e3 / launches             # average persistent launch, events on its stream
    bytes_per_launch = DECODE_ALGO_BYTES * L / launches
    achieved = bytes_per_launch / launch_s / 1e9
    value = L / (ms_step / 1e3)
    line = {
        "metric": "routed MoE-layer tokens/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "single-token decode, Qwen3-MoE layer (d_model 2048, d_ff 768, 128 Q8_0 "
                        "experts, Zipf-biased LinearGate, top-8); 48 distinct layers chained with "
                        "residual + RMSNorm per step",
            "tokens_per_layer_call": 1, "layers_per_step": L, "weights": "Q8_0",
            "algorithmic_bytes_per_layer_call": DECODE_ALGO_BYTES,
            "launches_per_step": launches,
        },
        "hbm_gbps": round(achieved, 1),
        "spread": dict(spread(step_reps), steps_per_repeat=max(1, a.steps // 10),
                       note="ms per step over further repeats after the timed region"),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": counter_traffic("decode_stack_q8_0", STACK_SRCS),
            "kernel": "decode_stack_kernel<Q8_0>",
            "avg_launch_us": round(launch_s * 1e6, 3),
            "algorithmic_bytes_per_launch": int(bytes_per_launch),
        },
    }
    extra = {}
    iters = max(3, min(20, a.steps // 10))
    if "toy" in want:
        extra["toy"] = bench_toy(torch, M, S, dev, stream, iters, cpu)
        print(f"[bench] toy: {extra['toy']['ms_per_call'] * 1e3:.2f} us per call", file=sys.stderr,
              flush=True)
    if "decode_per_layer" in want:
        bufs = [x0] + [torch.empty((1, D), dtype=torch.float32, device=dev) for _ in range(L)]

        def one_pass():
            for l in range(L):
                M.moe_layer(bufs[l], gates[l][0], gates[l][1], experts[l], K, bufs[l + 1],
                            flags=flags if l > 0 else M.F_RESIDUAL, ws=ws, stream=stream)

        pl_reps = graph_time_reps(torch, one_pass, stream, a.warmup, max(1, a.steps // 10), REPEATS)
        ms_pl = median_of(pl_reps)
        M.check_workspace(ws, stream=stream)
        diff = float((bufs[L][0] - outs[L - 1]).abs().max() / outs[L - 1].pow(2).mean().sqrt())
        extra["decode_per_layer"] = {
            "workload": "the same 48-layer step as 48 moe_layer calls (decode_stack_kernel<Q8_0>, one layer per launch)",
            "tokens_per_s": round(L / (ms_pl / 1e3), 1),
            "us_per_layer": round(ms_pl * 1e3 / L, 3),
            "hbm_gbps": round(DECODE_ALGO_BYTES / (ms_pl / 1e3 / L) / 1e9, 1),
            "hbm_frac": round(DECODE_ALGO_BYTES / (ms_pl / 1e3 / L) / 1e9 / HBM_PEAK_GBPS, 4),
            "max_rel_diff_vs_stack": diff,
            "spread": spread(pl_reps, L),
        }
        print(f"[bench] decode per layer: {ms_pl * 1e3 / L:.2f} us per layer call",
              file=sys.stderr, flush=True)
    if "decode_batch" in want:
        extra["decode_batch"] = bench_decode_batch(torch, M, S, dev, stream, iters, cpu)
        print(f"[bench] decode_batch: {extra['decode_batch']['ms_per_call'] * 1e3:.2f} us per layer",
              file=sys.stderr, flush=True)
    if "prefill_down" in want:
        extra["prefill_down"] = bench_prefill_down(torch, M, S, dev, stream, iters, cpu)
        pdn = extra["prefill_down"]
        print(f"[bench] prefill_down: {pdn['split_fp16']['ms_per_call'] * 1e3:.2f} "
              f"/ {pdn['fp16']['ms_per_call'] * 1e3:.2f} "
              f"/ banded {pdn['split_fp16_banded']['ms_per_call'] * 1e3:.2f} us per call",
              file=sys.stderr, flush=True)
    if "prefill_stack" in want:
        extra["prefill_stack"] = bench_prefill_stack(torch, M, S, dev, stream, arena, layers_np,
                                                     gates, max(2, iters // 4), cpu)
        print(f"[bench] prefill_stack: {extra['prefill_stack']['ms_per_pass']:.3f} ms per pass",
              file=sys.stderr, flush=True)
    if "attn_prep" in want:
        extra["attn_prep"] = bench_attn(torch, M, S, dev, stream, iters, cpu)
        print(f"[bench] attn_prep: {extra['attn_prep']['us_per_call']:.2f} us per token-layer",
              file=sys.stderr, flush=True)
    if extra:
        line["workloads"] = extra
    if cpu:
        line["cpu_baseline"] = cpu_decode(arena, layers_np, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
