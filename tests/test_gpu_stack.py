"""GPU parity of the 48-layer prefill stack (Qwen3-MoE geometry, Q8_0 experts).

2048 tokens x d_model 2048 run as two 1024-token microbatches through 48 layers,
each with its own LinearGate, Zipf bias and 128 experts (~30.8 GB of expert
blocks, all resident), with the residual add and the RMSNorm transition between
layers: o_l = in_l + MoE_l(in_l), in_{l+1} = rmsnorm(o_l).  The GPU runs free on
its own trajectory; at every layer the oracle's o_l and expert ids are compared
at sampled tokens (tokens are independent, so the oracle only follows those).
Sampled tokens are taken from seeded candidates whose fp64 trajectory keeps the
8th/9th router-logit gap at or above 1e-3 at every layer.
"""
import numpy as np
import pytest
import torch

import cases
import mixture_experts_routed_lineargate_amd as M
import moe_synth as S
from pins import rel_max_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CFG, L, T, MB, D, F, E, K = 5, 48, 2048, 1024, 2048, 768, 128, 8
TOL = 2e-3
N_CAND, N_KEEP = 6, 3


def test_stack_48_layers_two_microbatches():
    arena = S.device_arena(CFG, L, E, D, F, S.FMT_Q8_0, DEV)
    gates = cases.stack_layers(CFG, L, E, D, K)
    x0 = S.hidden(CFG, T, D)
    # candidates from both microbatches
    cand = np.sort(np.random.default_rng(55).choice(T, size=N_CAND, replace=False))
    print(f"\nstack: oracle trajectory of candidate tokens {cand.tolist()}", flush=True)
    ref = cases.stack_oracle(x0[cand], gates, arena, D, F, K, S.FMT_Q8_0)
    gap = np.min([cases.O.topk_gap(r["logits"], K) for r in ref], axis=0)
    keep = np.nonzero(gap >= cases.GAP)[0][:N_KEEP]
    assert keep.size >= 1, "no candidate keeps the gap rule through 48 layers"
    tok = cand[keep]
    print(f"stack: comparing tokens {tok.tolist()} (min gaps {gap[keep].tolist()})", flush=True)

    dG = [(torch.from_numpy(G).to(DEV), torch.from_numpy(b).to(DEV)) for G, b in gates]
    ex = [M.Experts.from_blobs(arena[l], D, F, S.FMT_Q8_0) for l in range(L)]
    xin = torch.from_numpy(x0).to(DEV)
    outs = torch.empty((L, T, D), dtype=torch.float32, device=DEV)
    ids = torch.empty((L, T, K), dtype=torch.int32, device=DEV)
    ws = M.workspace(MB, D, F, E, K, S.FMT_Q8_0, M.F_RESIDUAL | M.F_PRENORM)
    for mb in range(T // MB):
        sl = slice(mb * MB, (mb + 1) * MB)
        for l in range(L):
            src = xin[sl] if l == 0 else outs[l - 1, sl]
            flags = M.F_RESIDUAL | (M.F_PRENORM if l > 0 else 0)
            M.moe_layer(src, dG[l][0], dG[l][1], ex[l], K, outs[l, sl], flags=flags,
                        topk_ids=ids[l, sl], ws=ws)
    torch.cuda.synchronize()
    got = outs[:, torch.from_numpy(tok).to(DEV)].cpu().numpy()
    gids = ids[:, torch.from_numpy(tok).to(DEV)].cpu().numpy()
    worst = 0.0
    for l in range(L):
        r = ref[l]
        assert np.array_equal(gids[l], r["ids"][keep]), f"layer {l}: expert ids differ"
        err = rel_max_err(got[l], r["out"][keep])
        worst = max(worst, err)
        assert err <= TOL, f"layer {l}: max|d|/rms = {err:.3e}"
    assert torch.isfinite(outs).all()
    print(f"stack: worst per-layer max|d|/rms over 48 layers = {worst:.2e}", flush=True)
    del arena, outs
    torch.cuda.empty_cache()
