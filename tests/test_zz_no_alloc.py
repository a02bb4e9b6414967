"""moe_layer_noalloc (the library's static workspace, no allocation) against
moe_layer on a caller-owned workspace: three calls in a row on the same static
array with shrinking inputs (32 tokens on the small-batch kernels, then 5, then
a single token on the fused decode kernel), each bit-identical to moe_layer
with MOE_F_DETERMINISTIC and within the oracle's bound."""
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


def _outs(T, c):
    return dict(out=torch.empty((T, c.D), dtype=torch.float32, device=DEV),
                topk_ids=torch.empty((T, c.k), dtype=torch.int32, device=DEV),
                topk_w=torch.empty((T, c.k), dtype=torch.float32, device=DEV),
                expert_offsets=torch.empty(c.E + 1, dtype=torch.int32, device=DEV),
                sorted_rows=torch.empty(T * c.k, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("fmt", [S.FMT_Q4, S.FMT_Q8_0])
def test_noalloc_layer_matches_moe_layer(fmt):
    c = cases.router_case(f"noalloc{fmt}", 1100 + fmt, 32, 2048, 768, 128, 8, fmt, True, DEV)
    G, b = torch.from_numpy(c.G).to(DEV), torch.from_numpy(c.b).to(DEV)
    ex = M.Experts.from_blobs(c.arena, c.D, c.F, c.fmt)
    experts = c.oracle_experts()
    flags = M.F_RESIDUAL | M.F_DETERMINISTIC
    for T in (32, 5, 1):
        print(f"\nnoalloc: fmt {fmt}, T = {T}", flush=True)
        x = torch.from_numpy(np.ascontiguousarray(c.x[:T])).to(DEV)
        a, r = _outs(T, c), _outs(T, c)
        ws = M.workspace(T, c.D, c.F, c.E, c.k, c.fmt, flags)
        M.moe_layer(x, G, b, ex, c.k, ws=ws, flags=flags, **r)
        M.moe_layer_noalloc(x, G, b, ex, c.k, flags=flags, **a)
        torch.cuda.synchronize()
        M.check_workspace(ws)
        for key in a:
            ga, gr = a[key].cpu().numpy(), r[key].cpu().numpy()
            assert np.array_equal(ga.view(np.uint8), gr.view(np.uint8)), f"T={T}: {key} differs"
        ref = O.moe_layer(c.x[:T], c.G, c.b, experts, c.k, residual=True)
        assert np.array_equal(a["topk_ids"].cpu().numpy(), ref["ids"])
        err = rel_max_err(a["out"].cpu().numpy(), ref["out"])
        margins.record(f"noalloc T={T}", err)
        assert err <= 2e-3


def test_noalloc_rejects_too_large():
    c = cases.toy(DEV)
    big = 64
    x = torch.zeros((big, 2048), dtype=torch.float32, device=DEV)
    G = torch.zeros((2048, 128), dtype=torch.float32, device=DEV)
    arena = S.device_arena(3, 1, 128, 2048, 768, S.FMT_Q4, DEV)[0]
    ex = M.Experts.from_blobs(arena, 2048, 768, S.FMT_Q4)
    out = torch.empty((big, 2048), dtype=torch.float32, device=DEV)
    with pytest.raises(M.MoeError, match="status 6"):
        M.moe_layer_noalloc(x, G, None, ex, 8, out)
    del c
