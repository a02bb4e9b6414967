"""Seeded workloads shared by the GPU parity tests (inputs only; no layer arithmetic).

Geometry of the toy layer and of the Qwen3-MoE layer (d_model 2048, d_ff 768,
128 experts, top-8; evidence page, Model card).  Router inputs obey a gap rule
so the top-k set is unambiguous: the fp64 gap between the k-th and (k+1)-th
logit is at least 1e-3 (rows failing it are redrawn from their own seed
stream).  Expert arenas of the large geometry are drawn on the device; the
oracle reads back the bytes of the experts it needs.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import moe_synth as S
from oracle import moe_oracle as O

GAP = 1e-3
_POOL = None


def pool():
    """Threads for decoding experts in parallel (numpy releases the GIL in the
    decode); at most 16, the CPU share of one GPU."""
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0)))))
    return _POOL


def layer_experts(arena_l, D, F, fmt, experts=None):
    """The oracle's Experts for one layer's device arena [E][stride]: the bytes are
    copied to the host once, and the experts named in ``experts`` (all when None)
    are decoded up front by the oracle's own decoder on several threads."""
    host = arena_l.cpu().numpy()
    ex = O.Experts(lambda e: S.split_blob(host[e], D, F, fmt), fmt)
    todo = range(host.shape[0]) if experts is None else sorted(set(int(e) for e in experts))
    list(pool().map(ex.weights, todo))
    return ex


@dataclasses.dataclass
class Case:
    name: str
    T: int
    D: int
    F: int
    E: int
    k: int
    fmt: int
    x: np.ndarray = None          # [T][D] fp32 (None for the down-only operator)
    G: np.ndarray = None          # [D][E]
    b: np.ndarray = None          # [E] or None
    arena: object = None          # torch uint8 [E][stride] on the device
    h: np.ndarray = None          # down-only: [T*k][F]
    ids: np.ndarray = None        # down-only: [T][k] int32
    w: np.ndarray = None          # down-only: [T][k] fp32
    redraws: int = 0
    ref: object = None            # cached oracle result, when a test stores one

    def fetch(self, e: int):
        blob = self.arena[e].cpu().numpy()
        return S.split_blob(blob, self.D, self.F, self.fmt)

    def oracle_experts(self, prefetch=None):
        """The oracle's view of the case's experts; ``prefetch`` = expert ids to
        decode up front in parallel (large layers)."""
        if prefetch is not None:
            return layer_experts(self.arena, self.D, self.F, self.fmt, prefetch)
        return O.Experts(self.fetch, self.fmt)


def gap_rule(G, b, k, prenorm=False):
    """Accept rows whose router input (rmsnorm(x) when ``prenorm``) has an fp64
    k-th/(k+1)-th logit gap of at least GAP."""
    def accept(x):
        u = O.rmsnorm(x) if prenorm else x
        return O.topk_gap(O.router_logits(u, G, b), k) >= GAP
    return accept


def router_case(name, cfg, T, D, F, E, k, fmt, zipf: bool, device, host_experts=False,
                layer=0, prenorm=False) -> Case:
    import torch
    G = S.gate_matrix(cfg, D, E, layer=layer)
    b = S.zipf_bias(cfg, E, layer=layer) if zipf else None
    x = S.hidden(cfg, T, D, layer=layer)
    if prenorm:
        x *= np.float32(2.5)                      # exercise the normalisation
    red = S.redraw_until(x, cfg, gap_rule(G, b, k, prenorm), layer=layer) if k < E else np.zeros(T)
    if host_experts:
        arena = torch.from_numpy(S.expert_blobs(cfg, E, D, F, fmt, layer=layer)).to(device)
    else:
        arena = S.device_arena(cfg, 1, E, D, F, fmt, device)[0]
    return Case(name, T, D, F, E, k, fmt, x=x, G=G, b=b, arena=arena, redraws=int(red.sum()))


def toy(device):
    """16 tokens x d_model 256, 16 Q8_0 experts (256x128 / 128x256), top-2, no bias."""
    return router_case("toy", 1, 16, 256, 128, 16, 2, S.FMT_Q8_0, False, device, host_experts=True)


def decode(device):
    """1 token, Qwen geometry, Q8_0, Zipf-biased router."""
    return router_case("decode", 2, 1, 2048, 768, 128, 8, S.FMT_Q8_0, True, device)


def decode_batch(device):
    """32 tokens, Qwen geometry, 4-bit experts, Zipf-biased router."""
    return router_case("decode_batch", 3, 32, 2048, 768, 128, 8, S.FMT_Q4, True, device)


def prefill_down(device, T=1024):
    """Down projection only: T tokens routed top-8 over 128 experts, h ~ N(0,1), 4-bit W_down."""
    cfg, D, F, E, k = 4, 2048, 768, 128, 8
    G = S.gate_matrix(cfg, D, E)
    b = S.zipf_bias(cfg, E)
    xr = S.hidden(cfg, T, D)
    l = O.router_logits(xr, G, b)
    ids = O.select_topk(l, k)
    w = O.routing_weights(l, ids).astype(np.float32)
    h = S.generator(cfg, 0, S.ROLE_H).standard_normal((T * k, F), dtype=np.float32)
    arena = S.device_arena(cfg, 1, E, D, F, S.FMT_Q4, device, which=("down",))[0]
    return Case("prefill_down", T, D, F, E, k, S.FMT_Q4, arena=arena, h=h, ids=ids, w=w)


def stack_layers(cfg, L, E, D, k):
    """Per-layer LinearGate matrices and Zipf biases of a layer stack (independent seeds)."""
    return [(S.gate_matrix(cfg, D, E, layer=l), S.zipf_bias(cfg, E, layer=l)) for l in range(L)]


def stack_oracle(x_rows, gates, arena, D, F, k, fmt):
    """Oracle trajectory of token rows through every layer of the stack.

    Tokens are independent (no attention), so the trajectory of a token does not
    depend on which other tokens share its microbatch.  Each layer's experts are
    decoded up front on several threads (the oracle's own decoder; only the
    bytes' path into it is the harness's).  Returns the per-layer oracle results
    (``out`` = o_l, ``in`` = in_l, ``logits``, ``ids``, ``w``)."""
    def layers():
        for l, (G, b) in enumerate(gates):
            yield G, b, layer_experts(arena[l], D, F, fmt)

    def progress(l, r):
        if l % 8 == 7:
            print(f"  oracle: layer {l + 1}/{len(gates)} done", flush=True)
    return O.stack(x_rows, layers(), k, on_layer=progress)


def redraw_along_trajectory(x0, rows, cfg, gates, arena, D, F, k, fmt, n_alt=3, max_rounds=6):
    """Gap rule along the whole stack: redraw x0's rows (in place) until every
    layer of each row's fp64 trajectory keeps the k-th/(k+1)-th logit gap >= GAP.

    Row r's draws are x0[r] (attempt 0) then ``S.redraw_row(cfg, r, a, D)`` for
    a = 1, 2, ... (its own sub-seed stream); the row keeps its first draw whose
    trajectory holds the rule, which is what redrawing one attempt at a time
    would give.  Each round evaluates the next n_alt + 1 attempts of every
    pending row in one pass over the stack.  Returns ({row: oracle per-layer
    results of the kept draw}, {row: attempts used})."""
    rows = [int(r) for r in rows]
    ref, used = {}, {}
    pending = {r: 0 for r in rows}          # row -> first attempt of this round
    for _ in range(max_rounds):
        if not pending:
            break
        cand, who = [], []
        for r, a0 in pending.items():
            for a in range(a0, a0 + n_alt + 1):
                cand.append(x0[r] if a == 0 else S.redraw_row(cfg, r, a, D))
                who.append((r, a))
        res = stack_oracle(np.stack(cand).astype(np.float32), gates, arena, D, F, k, fmt)
        gap = np.min([O.topk_gap(l["logits"], k) for l in res], axis=0)
        nxt = {}
        for r, a0 in pending.items():
            ok = [i for i, (rr, a) in enumerate(who) if rr == r and gap[i] >= GAP]
            if ok:
                i = min(ok, key=lambda i: who[i][1])
                a = who[i][1]
                if a > 0:
                    x0[r] = S.redraw_row(cfg, r, a, D)
                ref[r] = [{key: l[key][i] for key in ("out", "in", "ids", "w", "logits")}
                          for l in res]
                used[r] = a
            else:
                nxt[r] = a0 + n_alt + 1
        pending = nxt
    if pending:
        raise RuntimeError(f"rows {sorted(pending)}: no draw keeps the gap rule")
    return ref, used
