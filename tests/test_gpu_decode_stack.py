"""GPU parity of the single-token decode stack (moe_decode_stack).

One token runs through a stack of Qwen3-MoE-geometry layers (d_model 2048, d_ff
768, 128 experts, Zipf-biased LinearGate routers, top-8), each with its residual
add, and the RMSNorm transition between layers.  The GPU runs free on its own
trajectory (one persistent launch per 24 layers); at every layer its o_l and
expert ids are compared with the oracle's trajectory.  Tokens are taken from
seeded candidates whose fp64 trajectory keeps the 8th/9th router-logit gap at or
above 1e-3 at every layer.
"""
import numpy as np
import pytest
import torch

import cases
import margins
import mixture_experts_routed_lineargate_amd as M
import moe_synth as S
from oracle import moe_oracle as O
from pins import rel_max_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D, F, E, K = 2048, 768, 128, 8
TOL = 2e-3


def pick_tokens(cfg, L, fmt, arena, gates, n_cand, n_keep, prenorm, seed):
    cand = S.hidden(cfg, n_cand, D, layer=seed)
    if prenorm:
        cand = cand * np.float32(3.0)
    x0 = O.rmsnorm(cand) if prenorm else cand
    ref = cases.stack_oracle(x0, gates, arena, D, F, K, fmt)
    gap = np.min([O.topk_gap(r["logits"], K) for r in ref], axis=0)
    keep = np.nonzero(gap >= cases.GAP)[0][:n_keep]
    assert keep.size >= 1, "no candidate keeps the gap rule through the stack"
    print(f"\ndecode stack: tokens {keep.tolist()} of {n_cand} keep the gap "
          f"(min gaps {gap[keep].tolist()})", flush=True)
    return cand, ref, keep


def run_stack(x, dG, ex, flags, ws):
    L = len(dG)
    layers = M.StackLayers([g for g, _ in dG], [b for _, b in dG], ex)
    outs = torch.full((L, D), float("nan"), dtype=torch.float32, device=DEV)
    ids = torch.full((L, K), -1, dtype=torch.int32, device=DEV)
    w = torch.zeros((L, K), dtype=torch.float32, device=DEV)
    M.moe_decode_stack(torch.from_numpy(x).to(DEV), layers, K, outs, flags=flags, topk_ids=ids,
                       topk_w=w, ws=ws)
    torch.cuda.synchronize()
    M.check_workspace(ws)
    return outs.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def check_trajectory(ref, t, outs, ids, w):
    worst = 0.0
    for l, r in enumerate(ref):
        assert np.array_equal(ids[l], r["ids"][t]), f"layer {l}: expert ids differ"
        assert np.abs(w[l] - r["w"][t]).max() <= 1e-5, f"layer {l}: routing weights"
        err = rel_max_err(outs[l][None], r["out"][t][None])
        worst = max(worst, err)
        assert err <= TOL, f"layer {l}: max|d|/rms = {err:.3e}"
    margins.record(f"token {t} through {len(ref)} layers", worst)
    return worst


def test_decode_stack_48_layers_q8_0():
    L = 48
    arena = S.device_arena(2, L, E, D, F, S.FMT_Q8_0, DEV)
    gates = cases.stack_layers(2, L, E, D, K)
    cand, ref, keep = pick_tokens(2, L, S.FMT_Q8_0, arena, gates, 4, 2, False, 600)
    dG = [(torch.from_numpy(G).to(DEV), torch.from_numpy(b).to(DEV)) for G, b in gates]
    ex = [M.Experts.from_blobs(arena[l], D, F, S.FMT_Q8_0) for l in range(L)]
    ws = M.workspace(1, D, F, E, K, S.FMT_Q8_0, M.F_PRENORM)
    first = None
    for t in keep:
        outs, ids, w = run_stack(cand[t], dG, ex, 0, ws)
        worst = check_trajectory(ref, t, outs, ids, w)
        print(f"decode stack Q8_0: token {t}: worst per-layer max|d|/rms = {worst:.2e}", flush=True)
        if first is None:
            first = (t, outs)
    # the single-layer kernel on the same workspace in between, then the stack again:
    # launch counters stay in step and the result is bit-identical
    t0, outs0 = first
    out1 = torch.empty((1, D), dtype=torch.float32, device=DEV)
    M.moe_layer(torch.from_numpy(cand[t0][None]).to(DEV), dG[0][0], dG[0][1], ex[0], K, out1,
                flags=M.F_RESIDUAL, ws=ws)
    again, _, _ = run_stack(cand[t0], dG, ex, 0, ws)
    assert np.array_equal(again.view(np.uint32), outs0.view(np.uint32)), "not bit-reproducible"
    del arena
    torch.cuda.empty_cache()


def test_decode_stack_q4_prenorm_crosses_launches():
    """30 4-bit layers: two launches (24 + 6); the first layer normalises its input."""
    L = 30
    arena = S.device_arena(3, L, E, D, F, S.FMT_Q4, DEV)
    gates = cases.stack_layers(3, L, E, D, K)
    cand, ref, keep = pick_tokens(3, L, S.FMT_Q4, arena, gates, 3, 1, True, 700)
    dG = [(torch.from_numpy(G).to(DEV), torch.from_numpy(b).to(DEV)) for G, b in gates]
    ex = [M.Experts.from_blobs(arena[l], D, F, S.FMT_Q4) for l in range(L)]
    ws = M.workspace(1, D, F, E, K, S.FMT_Q4, M.F_PRENORM)
    t = keep[0]
    outs, ids, w = run_stack(cand[t], dG, ex, M.F_PRENORM, ws)
    worst = check_trajectory(ref, t, outs, ids, w)
    print(f"decode stack Q4: token {t}: worst per-layer max|d|/rms = {worst:.2e}", flush=True)
    del arena
    torch.cuda.empty_cache()


def test_decode_stack_value_out_of_range_is_reported():
    """The stack sums each layer's output and the next router's logits in 64-bit
    fixed point.  An input value beyond that range (|x| >= 2^27 reaching the
    residual of layer 0) is not summed silently: the outputs from that layer on
    are NaN and moe_workspace_status reports MOE_E_RANGE (no wait times out).
    After a reset the workspace gives the same bits as a fresh one."""
    L = 3
    arena = S.device_arena(5, L, E, D, F, S.FMT_Q8_0, DEV)
    gates = cases.stack_layers(5, L, E, D, K)
    dG = [(torch.from_numpy(G).to(DEV), torch.from_numpy(b).to(DEV)) for G, b in gates]
    ex = [M.Experts.from_blobs(arena[l], D, F, S.FMT_Q8_0) for l in range(L)]
    layers = M.StackLayers([g for g, _ in dG], [b for _, b in dG], ex)
    x = S.hidden(5, 1, D)[0]
    bad = x.copy()
    bad[5] = np.float32(3.0e8)
    ws = M.workspace(1, D, F, E, K, S.FMT_Q8_0, M.F_PRENORM)
    outs = torch.zeros((L, D), dtype=torch.float32, device=DEV)
    print("\ndecode stack: an input beyond the fixed-point range", flush=True)
    M.moe_decode_stack(torch.from_numpy(bad).to(DEV), layers, K, outs, ws=ws)
    torch.cuda.synchronize()
    assert M.moe_workspace_status(ws) == M.MOE_E_RANGE
    o = outs.cpu().numpy()
    assert np.isnan(o[0]).any() and np.isnan(o[1:]).all(), "out-of-range input gave finite outputs"
    assert M.moe_workspace_status(ws, reset=True) == M.MOE_E_RANGE
    assert M.moe_workspace_status(ws) == M.MOE_OK
    got, _, _ = run_stack(x, dG, ex, 0, ws)
    fresh, _, _ = run_stack(x, dG, ex, 0, M.workspace(1, D, F, E, K, S.FMT_Q8_0, M.F_PRENORM))
    assert np.isfinite(got).all()
    assert np.array_equal(got.view(np.uint32), fresh.view(np.uint32)), "reset workspace differs"
    del arena
    torch.cuda.empty_cache()
