"""GPU parity of the attention-side primitives (moe_attn_prep): input RMSNorm with
gain, Q/K/V projection from block-quantized rows, grouped per-head Q/K RMSNorm,
RoPE and the F32 KV append, against the fp64 oracle on the same seeded inputs.
Bar: q, the appended k rows and the appended v rows each within
max|GPU - oracle| <= 2e-3 * RMS(oracle); cache rows no token writes keep their
sentinel bit for bit."""
import numpy as np
import pytest
import torch

import margins
import mixture_experts_routed_lineargate_amd as M
import moe_synth as S
from oracle import moe_oracle as O
from pins import rel_max_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3
SENTINEL = 12345.0


def run(cfg, T, D, nq, nkv, hd, fmt, pos, max_pos, theta=1e6, repeat=1):
    raw = S.qkv_weights(cfg, D, nq, nkv, hd, fmt)
    ga, gq, gk = S.attn_gain(cfg, D, 0), S.attn_gain(cfg, hd, 1), S.attn_gain(cfg, hd, 2)
    x = S.hidden(cfg, T, D) * np.float32(1.7)
    W = M.AttnWeights(torch.from_numpy(raw).to(DEV), torch.from_numpy(ga).to(DEV),
                      torch.from_numpy(gq).to(DEV), torch.from_numpy(gk).to(DEV), D, nq, nkv, hd, fmt)
    q = torch.full((T, nq, hd), float("nan"), dtype=torch.float32, device=DEV)
    kc = torch.full((max(max_pos, 1), nkv, hd), SENTINEL, dtype=torch.float32, device=DEV)
    vc = torch.full((max(max_pos, 1), nkv, hd), SENTINEL, dtype=torch.float32, device=DEV)
    ws = M.attn_workspace(T, W)
    outs = []
    for _ in range(repeat):
        M.moe_attn_prep(torch.from_numpy(x).to(DEV), W, torch.from_numpy(pos).to(DEV), q,
                        kc[:max_pos], vc[:max_pos], rope_theta=theta, ws=ws)
        torch.cuda.synchronize()
        M.check_workspace(ws)                 # raises if a head's wait gave up
        outs.append((q.cpu().numpy().copy(), kc.cpu().numpy()[:max_pos].copy(),
                     vc.cpu().numpy()[:max_pos].copy()))
    r = O.attn_prep(x, raw, fmt, ga, gq, gk, pos, theta, nq, nkv, hd)
    return outs, r


def check(outs, r, pos, max_pos, what):
    gq, gk, gv = outs[0]
    err = rel_max_err(gq, r["q"])
    margins.record(f"{what}: q", err)
    assert err <= TOL, f"q: {err:.3e}"
    ok = (pos >= 0) & (pos < max_pos)
    if ok.any():
        for name, g, ref in (("k", gk, r["k"]), ("v", gv, r["v"])):
            e = rel_max_err(g[pos[ok]], ref[ok])
            margins.record(f"{what}: {name}", e)
            assert e <= TOL, f"{name}: {e:.3e}"
    untouched = np.setdiff1d(np.arange(max_pos), pos[ok])
    assert (gk[untouched] == SENTINEL).all() and (gv[untouched] == SENTINEL).all()
    for later in outs[1:]:
        for a, b in zip(outs[0], later):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "not bit-reproducible"


@pytest.mark.parametrize("T,fmt", [(1, S.FMT_Q8_0), (1, S.FMT_Q4), (13, S.FMT_Q8_0), (40, S.FMT_Q4)])
def test_attn_prep_qwen_geometry(T, fmt):
    """d_model 2048, 32 q heads, 4 kv heads, head_dim 128 (5120 projection rows); one
    token (decode), a ragged 13-token block and 40 tokens; positions up to 8191."""
    pos = S.positions(40 + T, T, 8192)
    outs, r = run(40 + T, T, 2048, 32, 4, 128, fmt, pos, 8192, repeat=2)
    check(outs, r, pos, 8192, f"Qwen geometry T={T} fmt={fmt}")


@pytest.mark.parametrize("T,D,nq,nkv,hd,fmt", [
    (9, 160, 3, 1, 32, S.FMT_Q8_0),      # half a head of threads idle (hd/2 = 16)
    (3, 256, 2, 1, 256, S.FMT_Q4),       # two wavefronts per head
    (5, 3584, 8, 2, 64, S.FMT_Q8_0),     # largest d_model
])
def test_attn_prep_shapes(T, D, nq, nkv, hd, fmt):
    pos = S.positions(70 + T, T, 512)
    outs, r = run(70 + T, T, D, nq, nkv, hd, fmt, pos, 512)
    check(outs, r, pos, 512, f"D={D} heads={nq}/{nkv} hd={hd}")


def test_attn_prep_positions_outside_the_cache():
    """A position outside [0, max_pos) writes q only; the caches keep every row."""
    pos = np.array([3, -1, 64, 0, 63], dtype=np.int32)
    outs, r = run(90, 5, 256, 4, 2, 64, S.FMT_Q8_0, pos, 64)
    check(outs, r, pos, 64, "positions outside the cache")


def test_attn_prep_position_zero_is_identity_rope():
    """At position 0 RoPE is the identity: q equals the normalised projection."""
    pos = np.zeros(2, dtype=np.int32)
    pos[1] = 1
    outs, r = run(91, 2, 256, 2, 1, 64, S.FMT_Q4, pos, 8)
    check(outs, r, pos, 8, "position 0")
    qn = O.rmsnorm_gain(r["qkv"][:, :128].reshape(2, 2, 64), S.attn_gain(91, 64, 1))
    assert rel_max_err(outs[0][0][0], qn[0]) <= TOL
