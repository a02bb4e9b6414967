"""GPU parity: the HIP library against the fp64 CPU oracle on the same seeded inputs.

Bars: expert ids, expert_offsets and sorted_rows bit-exact; routing weights within
1e-5; every floating-point output within max|GPU - oracle| <= 2e-3 * RMS(oracle).
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
    M.check_workspace(ws)
    return {k: v.cpu().numpy() for k, v in
            dict(out=out, ids=ids, w=w, offsets=offs, sorted_rows=rows).items()}


def check_routing(g, r):
    assert np.array_equal(g["ids"], r["ids"]), "expert ids differ"
    assert np.abs(g["w"] - r["w"]).max() <= W_TOL
    assert np.array_equal(g["offsets"], r["offsets"])
    assert np.array_equal(g["sorted_rows"], r["sorted_rows"])


def check_out(got, ref, what="out"):
    err = rel_max_err(got, ref)
    margins.record(what, err)
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
    """Routing and layer output of every token against the oracle (ragged router
    tiles, partly filled GEMM tiles)."""
    c = cases.router_case(f"many{T}", 200 + T, T, 2048, 768, E, 8, fmt, True, DEV)
    g = run_layer(c, M.F_RESIDUAL)
    logits = O.router_logits(c.x, c.G, c.b)
    ids = O.select_topk(logits, c.k)
    assert np.array_equal(g["ids"], ids), "expert ids differ"
    assert np.abs(g["w"] - O.routing_weights(logits, ids)).max() <= W_TOL
    roff, rrows = O.group(g["ids"], c.E)
    assert np.array_equal(g["offsets"], roff) and np.array_equal(g["sorted_rows"], rrows)
    r = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(prefetch=np.unique(ids)), c.k, residual=True)
    check_out(g["out"], r["out"], f"T={T} E={E} every token")


@pytest.mark.parametrize("fmt", [S.FMT_Q4, S.FMT_Q8_0])
def test_weight_slice_experts_of_several_units(fmt):
    """64 tokens x top-8 = 512 routed rows, the most the weight-slice kernels take;
    the Zipf router gives several experts more than 32 rows (three or four 16-row
    units each).  Routing and every token's output against the oracle."""
    c = cases.router_case(f"units{fmt}", 264 + fmt, 64, 2048, 768, 128, 8, fmt, True, DEV)
    g = run_layer(c, M.F_RESIDUAL)
    logits = O.router_logits(c.x, c.G, c.b)
    ids = O.select_topk(logits, c.k)
    assert np.array_equal(g["ids"], ids), "expert ids differ"
    assert np.bincount(ids.ravel(), minlength=c.E).max() > 32, "no expert of three or more units"
    r = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(prefetch=np.unique(ids)), c.k, residual=True)
    check_out(g["out"], r["out"], f"64 tokens fmt={fmt} every token")


@pytest.fixture(scope="module")
def prefill_case():
    """1024-token Q8_0 layer at Qwen geometry, every token under the gap rule; the
    oracle runs the whole layer once (experts decoded in parallel)."""
    c = cases.router_case("prefill", 5, 1024, 2048, 768, 128, 8, S.FMT_Q8_0, True, DEV)
    ids = O.select_topk(O.router_logits(c.x, c.G, c.b), c.k)
    c.ref = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(prefetch=np.unique(ids)), c.k,
                        residual=True)
    return c


@pytest.mark.parametrize("flags", [M.F_RESIDUAL, M.F_RESIDUAL | M.F_FP16_ACT])
def test_prefill_layer_every_token(prefill_case, flags):
    """1024-token Q8_0 layer (grouped MFMA gate/up and down, 64-row tiles, two
    activation precisions): ids, weights, grouping and all 1024 x 2048 outputs."""
    c = prefill_case
    g = run_layer(c, flags)
    check_routing(g, c.ref)
    check_out(g["out"], c.ref["out"], f"1024-token layer flags={flags}")


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
    (6, 128, 64, 24, 12, 0),      # top-12: the ordered combine past its 8 preloaded slots
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
    assert M.moe_workspace_status(ws) == M.MOE_OK, "an exchange wait timed out"


def test_empty_input(toy_case):
    c = toy_case
    out = torch.full((1, c.D), 7.0, device=DEV)
    ws = M.workspace(1, c.D, c.F, c.E, c.k)
    x0 = torch.empty((0, c.D), dtype=torch.float32, device=DEV)
    M.moe_layer(x0, dev(c.G), None, experts_of(c), c.k, out, ws=ws)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


@pytest.mark.parametrize("T,k,E", [(2048, 8, 128), (1024, 8, 128), (1000, 8, 128), (513, 8, 100),
                                   (129, 8, 128), (128, 8, 128), (4096, 8, 256), (300, 8, 257),
                                   (1, 8, 128), (77, 2, 16)])
def test_group_large_and_invalid_ids(T, k, E):
    """Grouping against a stable argsort, with out-of-range ids (skipped).  1025 to
    32768 entries over at most 256 experts take the chunk-parallel kernel (one
    workgroup per 1024 entries, ragged last chunk included), the rest the
    single-workgroup one."""
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


def test_batch_layer_fp16_activations(batch_case):
    """32-token 4-bit layer on the weight-slice MFMA kernels with activations rounded
    to fp16 once (MOE_F_FP16_ACT) instead of two fp16 terms."""
    c = batch_case
    g = run_layer(c, M.F_RESIDUAL | M.F_FP16_ACT)
    r = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(), c.k, residual=True)
    check_routing(g, r)
    check_out(g["out"], r["out"], "32-token layer, fp16 activations")


# ---------------------------------------------------------------------------
# Dropped entries, masked experts, zero input
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,fmt", [(32, 1), (100, 0)])
def test_invalid_ids_through_expert_ffn(T, fmt):
    """Expert ids outside [0, E) handed to moe_group / moe_expert_ffn are dropped:
    the row adds nothing to out and its y row is zero.  T = 32 runs the weight-slice
    kernels (256 rows), T = 100 the grouped GEMM (800 rows); y is pre-filled with
    NaN, so a row the kernels skip would show."""
    c = cases.router_case(f"bad{T}", 300 + T, T, 2048, 768, 128, 8, fmt, True, DEV)
    ids, w, _ = O.route(c.x, c.G, c.b, c.k)
    bad = ids.copy()
    bad[3, 1] = c.E + 5
    bad[T - 1, 0] = -1
    bad[T // 2, 7] = c.E
    keep = (bad >= 0) & (bad < c.E)
    tx = dev(c.x)
    offs = torch.empty(c.E + 1, dtype=torch.int32, device=DEV)
    rows = torch.empty(T * c.k, dtype=torch.int32, device=DEV)
    ws = M.workspace(T, c.D, c.F, c.E, c.k, c.fmt)
    tid, tw = dev(bad.astype(np.int32)), dev(w.astype(np.float32))
    M.moe_group(tid, c.E, offs, rows, ws)
    y = torch.full((T * c.k, c.D), float("nan"), dtype=torch.float32, device=DEV)
    out = torch.empty((T, c.D), dtype=torch.float32, device=DEV)
    y2 = torch.full((T * c.k, c.D), float("nan"), dtype=torch.float32, device=DEV)
    M.moe_expert_ffn(tx, M.STAGE_FULL, experts_of(c), tid, tw, offs, rows, y=y, out=out,
                     flags=M.F_RESIDUAL, ws=ws)
    M.moe_expert_ffn(tx, M.STAGE_FULL, experts_of(c), tid, tw, offs, rows, y=y2, ws=ws)
    torch.cuda.synchronize()
    fixed = np.where(keep, bad, ids)                    # any valid id: its weight is 0 below
    yref = O.expert_outputs(c.x, fixed, c.oracle_experts())
    yref[~keep.ravel()] = 0.0
    ref = O.combine(yref, np.where(keep, w, 0.0), c.x)
    gy, gy2 = y.cpu().numpy(), y2.cpu().numpy()
    for g_y in (gy, gy2):
        assert np.isfinite(g_y).all()
        assert (g_y[~keep.ravel()] == 0).all()
    check_out(gy, yref, "y with dropped rows")
    assert np.array_equal(gy, gy2)
    check_out(out.cpu().numpy(), ref, "out with dropped rows")


@pytest.mark.parametrize("T", [1, 8, 40])
def test_masked_experts_negative_infinite_bias(T):
    """A -inf bias on E - k + 1 experts leaves k - 1 finite logits: those are
    selected, the k-th slot goes to the lowest-index masked expert with weight 0.
    T = 1 runs the fused decode kernel, T = 8 the one-launch small-batch routing,
    T = 40 the router + top-k pass (also through moe_route)."""
    c = cases.router_case(f"mask{T}", 500 + T, T, 2048, 768, 128, 8, S.FMT_Q8_0, True, DEV)
    rng = np.random.default_rng(T)
    b = c.b.copy()
    b[rng.choice(c.E, size=c.E - c.k + 1, replace=False)] = -np.inf
    mc = cases.Case(c.name, T, c.D, c.F, c.E, c.k, c.fmt, x=c.x, G=c.G, b=b, arena=c.arena)
    r = O.moe_layer(c.x, c.G, b, c.oracle_experts(), c.k, residual=True)
    assert (np.isfinite(np.take_along_axis(r["logits"], r["ids"].astype(np.int64), 1)).sum(1)
            == c.k - 1).all()
    g = run_layer(mc, M.F_RESIDUAL)
    check_routing(g, r)
    assert (g["w"][~np.isfinite(np.take_along_axis(r["logits"], r["ids"].astype(np.int64), 1))]
            == 0).all()
    check_out(g["out"], r["out"], "masked experts")
    ids = torch.empty((T, c.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, c.k), dtype=torch.float32, device=DEV)
    M.moe_route(dev(c.x), dev(c.G), dev(b), c.k, ids, w, M.workspace(T, c.D, c.F, c.E, c.k))
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.abs(w.cpu().numpy() - r["w"]).max() <= W_TOL


@pytest.mark.parametrize("T,fmt,flags", [(1, 0, M.F_RESIDUAL), (1, 1, M.F_PRENORM),
                                         (8, 1, M.F_RESIDUAL), (300, 0, M.F_RESIDUAL | M.F_PRENORM),
                                         (5, 0, M.F_RESIDUAL)])
def test_zero_input_gives_zero(T, fmt, flags):
    """x = 0: the ids are the top-k of the bias and out = 0 exactly (FFN(0) = 0 and
    the residual is 0), on the decode, small-batch, grouped and generic paths."""
    D, F, E = (2048, 768, 128) if T != 5 else (160, 96, 40)
    k = 8 if T != 5 else 5
    c = cases.router_case(f"zero{T}", 600 + T, T, D, F, E, k, fmt, True, DEV,
                          host_experts=(T == 5))
    z = np.zeros((T, D), np.float32)
    g = run_layer(c, flags, x=z)
    r = O.moe_layer(z, c.G, c.b, c.oracle_experts(), k, residual=True)
    check_routing(g, r)
    assert (g["out"] == 0).all()


# ---------------------------------------------------------------------------
# Invariants on the GPU
# ---------------------------------------------------------------------------

def scaled_down_arena(arena, D, F, fmt):
    """Copy of an expert arena with every W_down block scale doubled (fp16
    exponent + 1; every scale here is normal and far from the top)."""
    E = arena.shape[0]
    lay = S.blob_layout(D, F, fmt)
    bb = S.BLOCK_BYTES[fmt]
    a = arena.clone()
    reg = a[:, lay["down"]:lay["size"]].clone().reshape(E, -1, bb)
    bits = reg[..., 0].to(torch.int32) | (reg[..., 1].to(torch.int32) << 8)
    ex = (bits >> 10) & 0x1F
    assert bool(((ex >= 1) & (ex <= 29)).all())
    bits = bits + 0x400
    reg[..., 0] = (bits & 0xFF).to(torch.uint8)
    reg[..., 1] = (bits >> 8).to(torch.uint8)
    a[:, lay["down"]:lay["size"]] = reg.reshape(E, -1)
    return a


@pytest.mark.parametrize("T,D,F,E,k,fmt", [
    (1, 2048, 768, 128, 8, 0),      # fused decode kernel
    (32, 2048, 768, 128, 8, 1),     # weight-slice kernels
    (300, 2048, 768, 128, 8, 0),    # grouped GEMM
    (9, 160, 96, 40, 5, 1),         # generic kernels
])
def test_down_scale_linearity(T, D, F, E, k, fmt):
    """Doubling every W_down scale doubles the output (no residual,
    MOE_F_DETERMINISTIC): the scale enters every kernel as an exact factor, so the
    grouped and generic paths double bit for bit.  The single-token kernel sums
    the slots' outputs in fixed point with an absolute step of 2^-24, so there
    each of the 8 terms may round differently: |out2 - 2 out1| <= 8 * 2^-24, plus
    one fp32 rounding of the sum."""
    c = cases.router_case(f"lin{T}", 700 + T, T, D, F, E, k, fmt, True, DEV,
                          host_experts=(D != 2048))
    c2 = cases.Case(c.name, T, D, F, E, k, fmt, x=c.x, G=c.G, b=c.b,
                    arena=scaled_down_arena(c.arena, D, F, fmt))
    g1 = run_layer(c, M.F_DETERMINISTIC)
    g2 = run_layer(c2, M.F_DETERMINISTIC)
    assert np.array_equal(g1["ids"], g2["ids"])
    if T == 1 and D == 2048:
        diff = np.abs(g2["out"].astype(np.float64) - 2.0 * g1["out"].astype(np.float64))
        bound = 8 * 2.0 ** -24 + 2.0 ** -23 * np.abs(g2["out"].astype(np.float64))
        assert (diff <= bound).all(), f"worst {np.max(diff - bound):.3e} beyond the fixed-point bound"
    else:
        assert np.array_equal(g2["out"].view(np.uint32), (2 * g1["out"]).view(np.uint32))
    r = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(), k)
    check_out(g1["out"], r["out"], "linearity base layer")


@pytest.mark.parametrize("T,fmt", [(32, 1), (300, 0)])
def test_token_permutation(T, fmt):
    """Permuting the tokens permutes the ids, weights and outputs (each token's
    routing and FFN do not depend on its position in the batch)."""
    c = cases.router_case(f"perm{T}", 800 + T, T, 2048, 768, 128, 8, fmt, True, DEV)
    perm = np.random.default_rng(T).permutation(T)
    g = run_layer(c, M.F_RESIDUAL | M.F_DETERMINISTIC)
    gp = run_layer(c, M.F_RESIDUAL | M.F_DETERMINISTIC, x=np.ascontiguousarray(c.x[perm]))
    assert np.array_equal(gp["ids"], g["ids"][perm])
    assert np.array_equal(gp["w"], g["w"][perm])
    err = rel_max_err(gp["out"], g["out"][perm])
    print(f"\npermutation T={T}: max|d|/rms = {err:.2e} (0 = bit-identical)", flush=True)
    assert err <= 1e-6


# ---------------------------------------------------------------------------
# Block-format edge cases on every kernel family
# ---------------------------------------------------------------------------

SUBNORMAL, MAX_SCALE = 0x0123, 0x7BFF          # 2^-24 * 291 and 65504


def edge_arena(arena, D, F, fmt):
    """Copy of an expert arena with the block format's edge cases planted in every
    expert: in gate and up, zero-scale blocks, subnormal-scale blocks and (Q8_0)
    the code -128; in W_down, whole rows (output columns) with zero scales, with
    subnormal scales, and with the largest finite scale on their first block, plus
    scattered -128 codes.  Returns the arena and the column groups."""
    E = arena.shape[0]
    lay = S.blob_layout(D, F, fmt)
    bb = S.BLOCK_BYTES[fmt]
    a = arena.clone()
    cols = {"zero": np.arange(3, D, 97), "subnormal": np.arange(5, D, 89),
            "max": np.arange(7, D, 101)}
    for name, rows, n_in in (("gate", F, D), ("up", F, D), ("down", D, F)):
        nb = n_in // 32
        n = rows * nb * bb
        reg = a[:, lay[name]:lay[name] + n].clone().reshape(E, rows, nb, bb)
        idx = torch.arange(rows * nb, device=a.device).reshape(rows, nb)
        if fmt == S.FMT_Q8_0:
            reg[:, idx % 7 == 3, 2 + 17] = 0x80
        if name != "down":
            reg[:, idx % 13 == 5, 0:2] = 0
            reg[:, idx % 17 == 2, 0] = SUBNORMAL & 0xFF
            reg[:, idx % 17 == 2, 1] = SUBNORMAL >> 8
        else:
            z = torch.from_numpy(cols["zero"]).to(a.device)
            reg[:, z, :, 0:2] = 0
            sub = torch.from_numpy(cols["subnormal"]).to(a.device)
            pat = (torch.arange(nb, device=a.device) * 37 + 1) & 0x3FF     # 1 .. 1023
            reg[:, sub, :, 0] = (pat & 0xFF).to(torch.uint8)[None, None, :]
            reg[:, sub, :, 1] = (pat >> 8).to(torch.uint8)[None, None, :]
            mx = torch.from_numpy(cols["max"]).to(a.device)
            reg[:, mx, 0, 0] = MAX_SCALE & 0xFF
            reg[:, mx, 0, 1] = MAX_SCALE >> 8
        a[:, lay[name]:lay[name] + n] = reg.reshape(E, n)
    return a, cols


@pytest.mark.parametrize("T,D,F,E,k,fmt", [
    (1, 2048, 768, 128, 8, 0),      # fused decode kernel, Q8_0
    (1, 2048, 768, 128, 8, 1),      # fused decode kernel, 4-bit
    (32, 2048, 768, 128, 8, 0),     # weight-slice kernels
    (100, 2048, 768, 128, 8, 1),    # grouped GEMM
    (9, 160, 96, 40, 5, 0),         # generic kernels
])
def test_block_format_edge_cases(T, D, F, E, k, fmt):
    """Subnormal scales, zero-scale blocks, the largest finite scale and the code
    -128 against the oracle.  Output columns are compared by group, each against
    its own RMS: the subnormal columns are 10-100 times smaller than the rest and
    the max-scale columns ~1e6 times larger; zero-scale columns must be exactly 0
    (no residual)."""
    c = cases.router_case(f"edge{T}", 900 + T, T, D, F, E, k, fmt, True, DEV,
                          host_experts=(D != 2048))
    arena, cols = edge_arena(c.arena, D, F, fmt)
    ec = cases.Case(c.name, T, D, F, E, k, fmt, x=c.x, G=c.G, b=c.b, arena=arena)
    g = run_layer(ec, 0)
    r = O.moe_layer(c.x, c.G, c.b, ec.oracle_experts(), k)
    check_routing(g, r)
    assert (g["out"][:, cols["zero"]] == 0).all()
    special = np.concatenate(list(cols.values()))
    normal = np.setdiff1d(np.arange(D), special)
    check_out(g["out"][:, normal], r["out"][:, normal], "edge blocks: ordinary columns")
    check_out(g["out"][:, cols["subnormal"]], r["out"][:, cols["subnormal"]],
              "edge blocks: subnormal-scale columns")
    check_out(g["out"][:, cols["max"]], r["out"][:, cols["max"]], "edge blocks: max-scale columns")
    rs = np.sqrt((r["out"][:, cols["subnormal"]] ** 2).mean())
    rn = np.sqrt((r["out"][:, normal] ** 2).mean())
    rm = np.sqrt((r["out"][:, cols["max"]] ** 2).mean())
    assert 0 < rs < 0.5 * rn and rm > 1e3 * rn      # the groups really are that far apart


# ---------------------------------------------------------------------------
# A bounded exchange wait that gives up is reported, never silent
# ---------------------------------------------------------------------------

def test_forced_exchange_timeout(decode_case):
    """The fused decode kernels tag exchanged words with per-workgroup launch
    counters (bytes 4096.. of the workspace).  One counter put out of step from the
    host makes the words of that workgroup never match: every wait on them spends
    its bounded budget (the launch still ends), the error word is set, the outputs
    that depend on those words are NaN, and moe_workspace_status reports it.  After
    a reset the same workspace gives correct results again."""
    c = decode_case
    G, b, ex = dev(c.G), dev(c.b), experts_of(c)
    ws = M.workspace(1, c.D, c.F, c.E, c.k, c.fmt, M.F_PRENORM)
    out = torch.zeros((1, c.D), dtype=torch.float32, device=DEV)
    layers = M.StackLayers([G, G], [b, b], [ex, ex])
    outs = torch.zeros((2, c.D), dtype=torch.float32, device=DEV)
    for run in ("layer", "stack"):
        ws[4096 + 4 * 5:4096 + 4 * 6] = torch.tensor([7, 0, 0, 0], dtype=torch.uint8)
        print(f"\nforced timeout: {run} (a few seconds of bounded polling)", flush=True)
        if run == "layer":
            M.moe_layer(dev(c.x), G, b, ex, c.k, out, flags=M.F_RESIDUAL, ws=ws)
            res = out
        else:
            M.moe_decode_stack(dev(c.x[0]), layers, c.k, outs, ws=ws)
            res = outs
        torch.cuda.synchronize()
        assert M.moe_workspace_status(ws) == M.MOE_E_TIMEOUT
        assert torch.isnan(res).any(), "a timed-out launch returned finite outputs only"
        assert M.moe_workspace_status(ws, reset=True) == M.MOE_E_TIMEOUT
        assert M.moe_workspace_status(ws) == M.MOE_OK
        assert int(ws[:4 << 20].count_nonzero()) == 0
    M.moe_layer(dev(c.x), G, b, ex, c.k, out, flags=M.F_RESIDUAL, ws=ws)
    torch.cuda.synchronize()
    assert M.moe_workspace_status(ws) == M.MOE_OK
    r = O.moe_layer(c.x, c.G, c.b, c.oracle_experts(), c.k, residual=True)
    check_out(out.cpu().numpy(), r["out"], "after a reset")
