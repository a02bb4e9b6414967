"""GPU parity: the HIP library against the fp64 CPU oracle on the same seeded inputs.

Bars: expert ids, expert_offsets and sorted_rows bit-exact; routing weights within
1e-5; every floating-point output within max|GPU - oracle| <= 2e-3 * RMS(oracle).
"""
import numpy as np
import pytest
import torch

import cases
import mixture_experts_routed_lineargate_amd as M
import moe_synth as S
from oracle import moe_oracle as O
from pins import rel_max_err

pytestmark = pytest.mark.gpu
TOL = 2e-3
W_TOL = 1e-5
DEV = "cuda:0"


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def experts_of(case):
    return M.Experts.from_blobs(case.arena, case.D, case.F, case.fmt)


def run_layer(case, flags=0, x=None, T=None):
    x = case.x if x is None else x
    T = x.shape[0]
    tx = dev(x)
    out = torch.empty((T, case.D), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, case.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, case.k), dtype=torch.float32, device=DEV)
    offs = torch.empty(case.E + 1, dtype=torch.int32, device=DEV)
    rows = torch.empty(T * case.k, dtype=torch.int32, device=DEV)
    ws = M.workspace(T, case.D, case.F, case.E, case.k, case.fmt, flags)
    M.moe_layer(tx, dev(case.G), None if case.b is None else dev(case.b), experts_of(case),
                case.k, out, flags=flags, topk_ids=ids, topk_w=w, expert_offsets=offs,
                sorted_rows=rows, ws=ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in
            dict(out=out, ids=ids, w=w, offsets=offs, sorted_rows=rows).items()}


def check_routing(g, r):
    assert np.array_equal(g["ids"], r["ids"]), "expert ids differ"
    assert np.abs(g["w"] - r["w"]).max() <= W_TOL
    assert np.array_equal(g["offsets"], r["offsets"])
    assert np.array_equal(g["sorted_rows"], r["sorted_rows"])


def check_out(got, ref, what="out"):
    err = rel_max_err(got, ref)
    assert err <= TOL, f"{what}: max|d|/rms = {err:.3e}"
    return err


@pytest.fixture(scope="module")
def toy_case():
    return cases.toy(DEV)


@pytest.fixture(scope="module")
def decode_case():
    return cases.decode(DEV)


@pytest.fixture(scope="module")
def batch_case():
    return cases.decode_batch(DEV)


@pytest.mark.parametrize("name", ["toy_case", "decode_case", "batch_case"])
@pytest.mark.parametrize("flags", [0, M.F_RESIDUAL])
def test_layer_parity(name, flags, request):
    c = request.getfixturevalue(name)
    g = run_layer(c, flags)
    r = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(), c.k, residual=bool(flags & M.F_RESIDUAL))
    check_routing(g, r)
    check_out(g["out"], r["out"])


@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("rank", [7, 2])
def test_exact_tie_at_the_boundary(decode_case, T, rank):
    """Two experts with the same gate column and bias get bit-identical logits; when
    they tie for 8th place the lower index is selected (the router's tie-break).  The
    column of the expert ranked `rank` (0-based) is copied onto the next one: at 7
    the tied pair sits above the old 10th by at least the case's 1e-3 gap and the
    rest of the selection is unaffected; at 2 both stay selected and only the
    weights move.  T = 1 runs the fused single-token kernel and the decode stack
    (one layer), T = 4 the router partials + top-k pass."""
    c = decode_case
    x = np.repeat(c.x[:1], T, axis=0)
    order = np.argsort(-O.router_logits(x[:1], c.G, c.b)[0], kind="stable")
    e8, e9 = int(order[rank]), int(order[rank + 1])
    G2, b2 = c.G.copy(), c.b.copy()
    G2[:, e9] = G2[:, e8]
    b2[e9] = b2[e8]
    r = O.moe_layer(x, G2, b2, c.oracle_experts(), c.k, residual=True)
    if rank == c.k - 1:
        assert min(e8, e9) in r["ids"][0] and max(e8, e9) not in r["ids"][0]
    else:
        assert e8 in r["ids"][0] and e9 in r["ids"][0]
    tc = cases.Case(c.name, T, c.D, c.F, c.E, c.k, c.fmt, x=x, G=G2, b=b2, arena=c.arena)
    g = run_layer(tc, M.F_RESIDUAL)
    check_routing(g, r)
    check_out(g["out"], r["out"])
    if T == 1:
        layers = M.StackLayers([dev(G2)], [dev(b2)], [experts_of(c)])
        outs = torch.empty((1, c.D), dtype=torch.float32, device=DEV)
        ids = torch.empty((1, c.k), dtype=torch.int32, device=DEV)
        w = torch.empty((1, c.k), dtype=torch.float32, device=DEV)
        ws = M.workspace(1, c.D, c.F, c.E, c.k, c.fmt, M.F_PRENORM)
        M.moe_decode_stack(dev(x[0]), layers, c.k, outs, topk_ids=ids, topk_w=w, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), r["ids"])
        assert np.abs(w.cpu().numpy() - r["w"]).max() <= W_TOL
        check_out(outs.cpu().numpy(), r["out"])


@pytest.mark.parametrize("name", ["toy_case", "decode_case", "batch_case"])
def test_separate_calls_parity(name, request):
    c = request.getfixturevalue(name)
    T, k = c.T, c.k
    tx = dev(c.x)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    offs = torch.empty(c.E + 1, dtype=torch.int32, device=DEV)
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    y = torch.empty((T * k, c.D), dtype=torch.float32, device=DEV)
    out = torch.empty((T, c.D), dtype=torch.float32, device=DEV)
    out2 = torch.empty((T, c.D), dtype=torch.float32, device=DEV)
    ws = M.workspace(T, c.D, c.F, c.E, k, c.fmt)
    M.moe_route(tx, dev(c.G), None if c.b is None else dev(c.b), k, ids, w, ws)
    M.moe_group(ids, c.E, offs, rows, ws)
    M.moe_expert_ffn(tx, M.STAGE_FULL, experts_of(c), ids, w, offs, rows, y=y, ws=ws)
    M.moe_combine(y, w, out, residual=tx)
    M.moe_expert_ffn(tx, M.STAGE_FULL, experts_of(c), ids, w, offs, rows, out=out2,
                     flags=M.F_RESIDUAL, ws=ws)
    torch.cuda.synchronize()
    r = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(), k, residual=True)
    check_routing({"ids": ids.cpu().numpy(), "w": w.cpu().numpy(), "offsets": offs.cpu().numpy(),
                   "sorted_rows": rows.cpu().numpy()}, r)
    check_out(y.cpu().numpy(), r["y"], "y")
    check_out(out.cpu().numpy(), r["out"], "combine(y)")
    check_out(out2.cpu().numpy(), r["out"], "fused out")


@pytest.fixture(scope="module")
def down_case():
    c = cases.prefill_down(DEV)
    c.ref = O.down_combine(c.h, c.ids, c.w, c.oracle_experts())
    return c


@pytest.mark.parametrize("flags", [0, M.F_FP16_ACT, M.F_DETERMINISTIC])
def test_prefill_down_parity(down_case, flags):
    """1024 tokens x top-8 routed rows through the 4-bit down projection plus combine."""
    c = down_case
    T, k = c.T, c.k
    ids, w = dev(c.ids), dev(c.w)
    offs = torch.empty(c.E + 1, dtype=torch.int32, device=DEV)
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    out = torch.empty((T, c.D), dtype=torch.float32, device=DEV)
    ws = M.workspace(T, c.D, c.F, c.E, k, c.fmt)
    M.moe_group(ids, c.E, offs, rows, ws)
    M.moe_expert_ffn(dev(c.h), M.STAGE_DOWN, experts_of(c), ids, w, offs, rows, out=out,
                     flags=flags, ws=ws)
    torch.cuda.synchronize()
    roff, rrows = O.group(c.ids, c.E)
    assert np.array_equal(offs.cpu().numpy(), roff)
    assert np.array_equal(rows.cpu().numpy(), rrows)
    check_out(out.cpu().numpy(), c.ref)


def test_prefill_down_banded_is_bit_identical(down_case):
    """The banded tile walk (reuse-ordering page) changes only the order in which
    workgroups take tiles, so y and out match the default walk bit for bit, and
    the oracle like every other mode."""
    c = down_case
    T, k = c.T, c.k
    ids, w = dev(c.ids), dev(c.w)
    offs = torch.empty(c.E + 1, dtype=torch.int32, device=DEV)
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    ws = M.workspace(T, c.D, c.F, c.E, k, c.fmt)
    M.moe_group(ids, c.E, offs, rows, ws)
    res = []
    for flags in (0, M.F_BANDED):
        y = torch.full((T * k, c.D), float("nan"), dtype=torch.float32, device=DEV)
        out = torch.empty((T, c.D), dtype=torch.float32, device=DEV)
        M.moe_expert_ffn(dev(c.h), M.STAGE_DOWN, experts_of(c), ids, w, offs, rows, y=y, out=out,
                         flags=flags, ws=ws)
        torch.cuda.synchronize()
        res.append((y.cpu().numpy(), out.cpu().numpy()))
    assert np.array_equal(res[0][0].view(np.uint32), res[1][0].view(np.uint32))
    assert np.array_equal(res[0][1].view(np.uint32), res[1][1].view(np.uint32))
    check_out(res[1][1], c.ref)


@pytest.mark.parametrize("T,E,fmt", [
    (100, 100, 0),   # MFMA router with 100 experts and a ragged 32-token tile; 16-row GEMM tiles
    (70, 98, 1),     # 98 experts (not a multiple of 4): the FMA router for many tokens
    (300, 100, 1),   # 64-row GEMM tiles (some partly filled) with 100 experts
])
def test_many_token_shapes(T, E, fmt):
    """Routing of every token against the oracle's router; layer output on a sample
    of tokens that includes the ragged last router tile."""
    c = cases.router_case(f"many{T}", 200 + T, T, 2048, 768, E, 8, fmt, True, DEV)
    g = run_layer(c, M.F_RESIDUAL)
    logits = O.router_logits(c.x, c.G, c.b)
    ids = O.select_topk(logits, c.k)
    assert np.array_equal(g["ids"], ids), "expert ids differ"
    assert np.abs(g["w"] - O.routing_weights(logits, ids)).max() <= W_TOL
    roff, rrows = O.group(g["ids"], c.E)
    assert np.array_equal(g["offsets"], roff) and np.array_equal(g["sorted_rows"], rrows)
    rng = np.random.default_rng(T)
    sample = np.unique(np.concatenate([rng.choice(T, size=10, replace=False),
                                       np.arange(T - 3, T)]))
    r = O.moe_layer(c.x[sample], c.G, c.b, c.oracle_experts(), c.k, residual=True)
    check_out(g["out"][sample], r["out"])


def test_prefill_layer_sampled_tokens():
    """1024-token Q8_0 layer at Qwen geometry; the oracle checks a sample of tokens
    (tokens are independent through one layer)."""
    c = cases.router_case("prefill", 5, 1024, 2048, 768, 128, 8, S.FMT_Q8_0, True, DEV)
    g = run_layer(c, M.F_RESIDUAL)
    sample = np.random.default_rng(0).choice(c.T, size=40, replace=False)
    sample.sort()
    r = O.moe_layer(c.x[sample], c.G, c.b, c.oracle_experts(), c.k, residual=True)
    assert np.array_equal(g["ids"][sample], r["ids"])
    assert np.abs(g["w"][sample] - r["w"]).max() <= W_TOL
    # grouping of the full routing, checked against the oracle's grouping of the GPU ids
    roff, rrows = O.group(g["ids"], c.E)
    assert np.array_equal(g["offsets"], roff) and np.array_equal(g["sorted_rows"], rrows)
    check_out(g["out"][sample], r["out"])


@pytest.mark.parametrize("T,D,F,E,k,fmt", [
    (5, 256, 128, 16, 2, 0),      # ragged toy
    (37, 2048, 768, 128, 8, 1),   # ragged beyond a 32-token tile, 4-bit
    (3, 2048, 768, 128, 1, 0),    # top-1
    (17, 2048, 768, 64, 4, 0),    # odd small batch, 64 experts, top-4 (one-launch routing)
    (9, 2048, 768, 128, 8, 1),    # one-launch routing: a full 8-token group and a 1-token group
    (32, 2048, 768, 100, 8, 1),   # 100 experts (one-launch routing, non-power-of-two grouping)
    (4, 96, 64, 1, 1, 1),         # one expert, top-1: a dense SwiGLU FFN
    (7, 64, 32, 6, 6, 0),         # every expert selected
    (9, 160, 96, 40, 5, 1),       # odd geometry (generic kernels)
])
def test_edge_shapes(T, D, F, E, k, fmt):
    c = cases.router_case(f"edge{T}", 100 + T, T, D, F, E, k, fmt, E > 8, DEV, host_experts=True)
    g = run_layer(c, M.F_RESIDUAL)
    r = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(), k, residual=True)
    check_routing(g, r)
    check_out(g["out"], r["out"])


def test_prenorm_flag():
    c = cases.router_case("toy_prenorm", 7, 16, 256, 128, 16, 2, S.FMT_Q8_0, False, DEV,
                          host_experts=True, prenorm=True)
    g = run_layer(c, M.F_RESIDUAL | M.F_PRENORM)
    r = O.moe_layer(O.rmsnorm(c.x), c.G, c.b, c.oracle_experts(), c.k, residual=True)
    check_routing(g, r)
    check_out(g["out"], r["out"])


@pytest.mark.parametrize("fmt", [S.FMT_Q8_0, S.FMT_Q4])
@pytest.mark.parametrize("flags", [0, M.F_RESIDUAL, M.F_RESIDUAL | M.F_PRENORM])
def test_single_token_layer(fmt, flags):
    """Single-token Qwen-geometry layer (the fused one-launch decode path), both formats."""
    pre = bool(flags & M.F_PRENORM)
    c = cases.router_case(f"decode{fmt}", 20 + fmt, 1, 2048, 768, 128, 8, fmt, True, DEV,
                          prenorm=pre)
    g = run_layer(c, flags)
    u = O.rmsnorm(c.x) if pre else c.x
    r = O.moe_layer(u, c.G, c.b, c.oracle_experts(), c.k, residual=bool(flags & M.F_RESIDUAL))
    check_routing(g, r)
    check_out(g["out"], r["out"])


def test_single_token_repeated_calls(decode_case):
    """Many consecutive one-launch decode calls on one workspace (its barrier counter keeps
    running across calls): every call matches the oracle and no wait timed out."""
    c = decode_case
    ws = M.workspace(1, c.D, c.F, c.E, c.k, c.fmt, M.F_RESIDUAL)
    G, b, ex = dev(c.G), dev(c.b), experts_of(c)
    experts = c.oracle_experts()
    out = torch.empty((1, c.D), dtype=torch.float32, device=DEV)
    for rep in range(6):
        x = S.hidden(400 + rep, 1, c.D)
        S.redraw_until(x, 400 + rep, cases.gap_rule(c.G, c.b, c.k))
        M.moe_layer(dev(x), G, b, ex, c.k, out, flags=M.F_RESIDUAL, ws=ws)
        torch.cuda.synchronize()
        r = O.moe_layer(x, c.G, c.b, experts, c.k, residual=True)
        check_out(out.cpu().numpy(), r["out"], f"call {rep}")
    assert int(ws[64:68].view(torch.int32).item()) == 0, "grid barrier timed out"


def test_empty_input(toy_case):
    c = toy_case
    out = torch.full((1, c.D), 7.0, device=DEV)
    ws = M.workspace(1, c.D, c.F, c.E, c.k)
    x0 = torch.empty((0, c.D), dtype=torch.float32, device=DEV)
    M.moe_layer(x0, dev(c.G), None, experts_of(c), c.k, out, ws=ws)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


@pytest.mark.parametrize("T,k,E", [(2048, 8, 128), (1000, 8, 128), (513, 8, 100), (129, 8, 128),
                                   (1, 8, 128), (77, 2, 16)])
def test_group_large_and_invalid_ids(T, k, E):
    """Grouping against a stable argsort, with out-of-range ids (skipped).  1025 to
    8192 entries over at most 128 experts take the single-pass kernel, the rest
    the chunked one."""
    rng = np.random.default_rng(21 + T)
    p = np.exp(-1.1 * np.log(np.arange(1, E + 1)))
    p /= p.sum()
    ids = np.stack([np.sort(rng.choice(E, size=k, replace=False, p=p)) for _ in range(T)])
    ids = ids.astype(np.int32)
    for bad in (False, True):
        if bad:
            ids[min(3, T - 1), 1] = E + 5
            ids[min(100, T - 1), 0] = -1
        offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
        M.moe_group(dev(ids), E, offs, rows)
        torch.cuda.synchronize()
        valid = (ids >= 0) & (ids < E)
        flat = ids.ravel()
        ref_rows = np.argsort(np.where(valid.ravel(), flat, E + 1), kind="stable")[:valid.sum()]
        counts = np.bincount(flat[valid.ravel()], minlength=E)
        assert np.array_equal(offs.cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]))
        assert np.array_equal(rows.cpu().numpy()[:valid.sum()], ref_rows)


def test_rmsnorm_parity():
    x = S.hidden(9, 33, 2048) * 2.5
    out = torch.empty_like(dev(x))
    M.moe_rmsnorm(dev(x), out, 1e-6)
    torch.cuda.synchronize()
    check_out(out.cpu().numpy(), O.rmsnorm(x, 1e-6))
    err = np.abs(out.cpu().numpy() - O.rmsnorm(x, 1e-6)).max()
    assert err < 1e-5


def test_deterministic_repeat(batch_case):
    a = run_layer(batch_case, M.F_DETERMINISTIC)
    b = run_layer(batch_case, M.F_DETERMINISTIC)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_graph_replay_with_changed_inputs(batch_case):
    """Capture moe_layer once, change x in place, replay, compare every replay with the oracle."""
    c = batch_case
    T = c.T
    tx = dev(c.x)
    out = torch.zeros((T, c.D), dtype=torch.float32, device=DEV)
    ws = M.workspace(T, c.D, c.F, c.E, c.k, c.fmt)
    G, b, ex = dev(c.G), dev(c.b), experts_of(c)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        M.moe_layer(tx, G, b, ex, c.k, out, ws=ws, stream=stream)   # warm-up outside capture
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        M.moe_layer(tx, G, b, ex, c.k, out, ws=ws, stream=stream)
    experts = c.oracle_experts()
    for rep in range(3):
        x = S.hidden(300 + rep, T, c.D)
        S.redraw_until(x, 300 + rep, cases.gap_rule(c.G, c.b, c.k))
        tx.copy_(torch.from_numpy(x))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        r = O.moe_layer(x, c.G, c.b, experts, c.k)
        check_out(out.cpu().numpy(), r["out"], f"replay {rep}")
