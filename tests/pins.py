"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes the oracle module ``O`` (``oracle.moe_oracle``) so the
mutation tests can hand in a copy with a planted mistake and check that some
pin catches it.  Sources of truth used here:

* figures printed on the MER evidence page (``golden/page_numbers.json``);
* closed forms of the block formats, checked exhaustively against Python's
  ``struct`` fp16 decoder and numpy's float16;
* library routines the layer reduces to in special cases (torch float64
  matmul / silu / rms_norm, scipy softmax, numpy stable argsort);
* brute force on tiny inputs (``oracle.scalar``: subset search, Python loops);
* invariants (renormalisation, shift invariance, linearity, equivariance).
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

import moe_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_numbers():
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Page figures
# ---------------------------------------------------------------------------

def pin_page_expert_size(O):
    """Q8_0 expert bytes at the stated geometry match the page's bytes-per-miss and cache sizes."""
    pg = _page_numbers()
    geo = pg["geometry"]
    blob = O.expert_bytes(geo["d_model"], geo["d_ff"], O.Q8_0)
    for r in pg["cache_tradeoff"]["rows"]:
        per_miss = r["data_read_gb"] * 1e9 / r["misses"]
        assert abs(per_miss / blob - 1) < 5e-3, (per_miss, blob)
    for r in pg["synthetic_cache_matrix"]["rows"] + pg["cache_tradeoff"]["rows"]:
        gib = r["slots"] * blob / 2**30
        assert abs(gib / r["raw_cache_gib"] - 1) < 3e-3, (r, gib)


def pin_page_accesses():
    """One expert access per (forward, layer, selected expert): 158 x 48 x 8 reproduces the hit rates."""
    pg = _page_numbers()
    geo, meth = pg["geometry"], pg["methodology"]
    assert meth["prompt_tokens"] + meth["completion_tokens"] - 1 == meth["forwards"]
    acc = meth["forwards"] * geo["layers"] * geo["top_k"]
    for r in pg["cache_tradeoff"]["rows"]:
        hit = 100 * (1 - r["misses"] / acc)
        digits = len(str(r["hit_rate_pct"]).split(".")[1])
        assert round(hit, digits) == r["hit_rate_pct"], (hit, r)
    for r in pg["synthetic_cache_matrix"]["rows"]:
        assert round(r["misses"] / (1 - r["hit_rate_pct"] / 100)) == 80000


# ---------------------------------------------------------------------------
# Block formats
# ---------------------------------------------------------------------------

def _finite_fp16_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    return bits[((bits >> 10) & 0x1F) != 31]


def pin_fp16_decoder(O):
    bits = np.arange(65536, dtype=np.uint32)
    got = O.fp16_bits_to_f64(bits)
    ref_np = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    fin = np.isfinite(ref_np)
    assert np.array_equal(got[fin], ref_np[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref_np))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref_np) & (ref_np > 0))
    for b in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xC000, 0x3555):
        assert got[b] == struct.unpack("<e", struct.pack("<H", b))[0]


def pin_q8_0_exhaustive(O):
    """Every finite fp16 scale x every int8 code: decoded value == d*q exactly."""
    scales = _finite_fp16_patterns()
    q = np.arange(-128, 128, dtype=np.int64)           # 256 codes = 8 blocks per scale
    n = scales.size
    raw = np.zeros((n, 8, 34), dtype=np.uint8)
    raw[:, :, 0] = (scales & 0xFF)[:, None]
    raw[:, :, 1] = (scales >> 8)[:, None]
    raw[:, :, 2:] = (q.reshape(8, 32) & 0xFF).astype(np.uint8)[None]
    got = O.decode_rows(raw.reshape(n, 8 * 34), O.Q8_0)
    d = scales.astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.array_equal(got, d[:, None] * q[None, :].astype(np.float64))


def pin_q4_exhaustive(O):
    """Every finite fp16 scale x every nibble in both halves: value == d*(q-8) exactly."""
    scales = _finite_fp16_patterns()
    n = scales.size
    raw = np.zeros((n, 18), dtype=np.uint8)
    raw[:, 0] = scales & 0xFF
    raw[:, 1] = scales >> 8
    lo = np.arange(16, dtype=np.uint8)                  # bytes 0..15: low nibble = i
    hi = (15 - np.arange(16)).astype(np.uint8)          # high nibble = 15 - i
    raw[:, 2:] = (lo | (hi << 4))[None]
    got = O.decode_rows(raw, O.Q4)
    d = scales.astype(np.uint16).view(np.float16).astype(np.float64)
    expect_q = np.empty(32)
    expect_q[0::2] = lo.astype(np.float64) - 8
    expect_q[1::2] = hi.astype(np.float64) - 8
    assert np.array_equal(got, d[:, None] * expect_q[None, :])


def _exact_matrix(rng, n_in, n_out, fmt):
    """A [in][out] matrix with exactly known values and its block bytes, built by hand."""
    nb = n_in // 32
    e = rng.integers(-9, -4, size=(n_out, nb))          # scales 2^e, exact in fp16
    d = np.ldexp(1.0, e)
    if fmt == 0:
        q = rng.integers(-128, 128, size=(n_out, nb, 32))
        vals = d[..., None] * q
        raw = np.zeros((n_out, nb, 34), dtype=np.uint8)
        raw[..., 2:] = (q & 0xFF).astype(np.uint8)
    else:
        q = rng.integers(0, 16, size=(n_out, nb, 32))
        vals = d[..., None] * (q - 8)
        raw = np.zeros((n_out, nb, 18), dtype=np.uint8)
        raw[..., 2:] = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    h = d.astype(np.float16).view(np.uint16)
    raw[..., 0] = h & 0xFF
    raw[..., 1] = h >> 8
    return vals.reshape(n_out, n_in).T.copy(), raw.reshape(n_out, -1)


def pin_matrix_orientation(O):
    rng = np.random.default_rng(11)
    for fmt in (O.Q8_0, O.Q4):
        W, raw = _exact_matrix(rng, 96, 40, fmt)
        assert np.array_equal(O.dequant_matrix(raw, fmt), W)


def pin_encoder_roundtrip(O):
    """The fixture encoders invert to within half a step under the oracle's decoder."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    for fmt, qmax in ((O.Q8_0, 127), (O.Q4, 7)):
        raw = S.quantize(w, fmt)
        back = O.decode_rows(raw, fmt)
        step = np.abs(w.reshape(64, 8, 32)).max(axis=2) / qmax
        err = np.abs(back - w).reshape(64, 8, 32).max(axis=2)
        assert np.all(err <= 0.5 * step * (1 + 2e-3) + 1e-12)


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def pin_topk_bruteforce(O):
    from oracle import scalar
    rng = np.random.default_rng(3)
    for trial in range(300):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-3, 4, size=(1, E)).astype(np.float64)   # many exact ties
        if trial % 2:
            l = rng.standard_normal((1, E))
        got = O.select_topk(l, k)[0].tolist()
        assert got == scalar.topk_bruteforce(l[0].tolist(), k), (l, k, got)


def pin_tie_break_zero_gate(O):
    for E, k in ((16, 2), (128, 8), (8, 8), (5, 1)):
        x = np.random.default_rng(E).standard_normal((3, 32))
        ids, w, _ = O.route(x, np.zeros((32, E)), np.zeros(E), k)
        assert (ids == np.arange(k)[None]).all()
        assert (w == 1.0 / k).all()


def pin_weights_closed_form(O):
    rng = np.random.default_rng(8)
    l = rng.standard_normal((50, 20)) * 3
    ids = O.select_topk(l, 5)
    w = O.routing_weights(l, ids)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    # w_j = 1 / sum_j' exp(l_j' - l_j)
    ref = 1.0 / np.exp(sel[:, None, :] - sel[:, :, None]).sum(axis=2)
    assert np.allclose(w, ref, rtol=1e-13, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # a shift of all logits changes nothing
    assert (O.select_topk(l + 7.25, 5) == ids).all()
    assert np.allclose(O.routing_weights(l + 7.25, ids), w, rtol=1e-13)
    # selected weights are ordered like their logits
    assert np.all((np.diff(sel, axis=1) > 0) == (np.diff(w, axis=1) > 0))


def pin_full_selection_is_softmax(O):
    """k == E: the weights are the plain softmax (scipy) of the logits."""
    from scipy.special import softmax
    rng = np.random.default_rng(9)
    l = rng.standard_normal((10, 6)) * 2
    ids = O.select_topk(l, 6)
    assert (ids == np.arange(6)[None]).all()
    assert np.allclose(O.routing_weights(l, ids), softmax(l, axis=1), rtol=1e-13, atol=0)


def pin_router_logits(O):
    """Logits are x G + b with G as [D][E] (checked against torch float64 matmul)."""
    import torch
    rng = np.random.default_rng(10)
    x = rng.standard_normal((7, 48)).astype(np.float32)
    G = rng.standard_normal((48, 12)).astype(np.float32)
    b = rng.standard_normal(12).astype(np.float32)
    ref = (torch.from_numpy(x).double() @ torch.from_numpy(G).double() + torch.from_numpy(b).double()).numpy()
    assert np.allclose(O.router_logits(x, G, b), ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# Grouping
# ---------------------------------------------------------------------------

def pin_grouping(O):
    rng = np.random.default_rng(12)
    for T, k, E in ((1, 8, 128), (16, 2, 16), (300, 8, 128), (64, 3, 5)):
        ids = np.stack([np.sort(rng.choice(E, size=k, replace=False)) for _ in range(T)]).astype(np.int32)
        off, rows = O.group(ids, E)
        assert np.array_equal(rows, np.argsort(ids.ravel(), kind="stable"))
        assert off[0] == 0 and off[-1] == T * k
        assert np.array_equal(np.diff(off), np.bincount(ids.ravel(), minlength=E))


# ---------------------------------------------------------------------------
# Expert FFN and the whole layer
# ---------------------------------------------------------------------------

def _experts_from(mats, fmt, O):
    return O.Experts(lambda e: mats[e], fmt)


def pin_dense_reduction(O):
    """E = 1, k = 1: the layer is one dense SwiGLU FFN (torch float64 silu/matmul)."""
    import torch
    import torch.nn.functional as Fn
    rng = np.random.default_rng(13)
    D, F_ = 64, 96
    for fmt in (O.Q8_0, O.Q4):
        Wg, rg = _exact_matrix(rng, D, F_, fmt)
        Wu, ru = _exact_matrix(rng, D, F_, fmt)
        Wd, rd = _exact_matrix(rng, F_, D, fmt)
        x = rng.standard_normal((5, D)).astype(np.float32)
        G = rng.standard_normal((D, 1)).astype(np.float32)
        r = O.moe_layer(x, G, None, _experts_from({0: (rg, ru, rd)}, fmt, O), 1)
        tx = torch.from_numpy(x).double()
        ref = (Fn.silu(tx @ torch.from_numpy(Wg)) * (tx @ torch.from_numpy(Wu))) @ torch.from_numpy(Wd)
        assert np.allclose(r["out"], ref.numpy(), rtol=1e-12, atol=1e-12)
        assert (r["ids"] == 0).all() and (r["w"] == 1.0).all()
        r2 = O.moe_layer(x, G, None, _experts_from({0: (rg, ru, rd)}, fmt, O), 1, residual=True)
        assert np.allclose(r2["out"], ref.numpy() + x, rtol=1e-12, atol=1e-12)


def pin_all_experts_mixture(O):
    """k = E: out = sum_e softmax(l)_e FFN_e(x) (scipy softmax, torch float64 FFNs)."""
    import torch
    import torch.nn.functional as Fn
    from scipy.special import softmax
    rng = np.random.default_rng(14)
    D, F_, E = 32, 64, 3
    mats, dense = {}, {}
    for e in range(E):
        Wg, rg = _exact_matrix(rng, D, F_, 0)
        Wu, ru = _exact_matrix(rng, D, F_, 0)
        Wd, rd = _exact_matrix(rng, F_, D, 0)
        mats[e] = (rg, ru, rd)
        dense[e] = tuple(torch.from_numpy(m) for m in (Wg, Wu, Wd))
    x = rng.standard_normal((4, D)).astype(np.float32)
    G = (rng.standard_normal((D, E)) * 0.3).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    r = O.moe_layer(x, G, b, _experts_from(mats, 0, O), E)
    tx = torch.from_numpy(x).double()
    p = softmax(x.astype(np.float64) @ G.astype(np.float64) + b, axis=1)
    ref = np.zeros((4, D))
    for e in range(E):
        Wg, Wu, Wd = dense[e]
        ref += p[:, e:e + 1] * ((Fn.silu(tx @ Wg) * (tx @ Wu)) @ Wd).numpy()
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-13)


def pin_zero_input(O):
    """x = 0: ids are the top-k of the bias and out = 0 exactly."""
    from oracle import scalar
    D, F_, E, k = 64, 32, 16, 4
    blobs = S.expert_blobs(1, E, D, F_, S.FMT_Q8_0)
    ex = _experts_from({e: S.split_blob(blobs[e], D, F_, 0) for e in range(E)}, 0, O)
    b = S.zipf_bias(1, E)
    G = S.gate_matrix(1, D, E)
    r = O.moe_layer(np.zeros((2, D), np.float32), G, b, ex, k)
    assert (r["out"] == 0).all()
    assert r["ids"][0].tolist() == scalar.topk_bruteforce(b.astype(np.float64).tolist(), k)


def pin_scalar_bruteforce(O, T=8):
    """The vectorised oracle equals the Python-loop oracle on the toy geometry."""
    from oracle import scalar
    D, F_, E, k = 256, 128, 16, 2
    x = S.hidden(1, T, D)
    G = S.gate_matrix(1, D, E)
    for fmt in (S.FMT_Q8_0, S.FMT_Q4):
        blobs = S.expert_blobs(1, E, D, F_, fmt)
        mats = {e: S.split_blob(blobs[e], D, F_, fmt) for e in range(E)}
        r = O.moe_layer(x, G, None, _experts_from(mats, fmt, O), k, residual=(fmt == 1))
        s = scalar.layer(x, G, None, mats, fmt, k, residual=(fmt == 1))
        assert r["ids"].tolist() == s["ids"]
        assert np.allclose(r["w"], np.array(s["w"]), rtol=1e-12, atol=0)
        ref = np.array(s["out"])
        assert np.abs(r["out"] - ref).max() <= 1e-12 * np.sqrt((ref ** 2).mean())
        assert r["offsets"].tolist() == s["offsets"]
        assert r["sorted_rows"].tolist() == s["sorted_rows"]


def pin_linearity(O):
    """Doubling every W_down scale (fp16 exponent + 1) doubles the output exactly."""
    D, F_, E, k = 64, 32, 8, 2
    blobs = S.expert_blobs(2, E, D, F_, S.FMT_Q8_0)
    mats = {e: S.split_blob(blobs[e], D, F_, 0) for e in range(E)}
    mats2 = {}
    for e, (g, u, d) in mats.items():
        d2 = d.copy().reshape(D, -1, 34)
        bits = d2[..., 0].astype(np.uint32) | (d2[..., 1].astype(np.uint32) << 8)
        assert (((bits >> 10) & 0x1F) < 30).all() and (((bits >> 10) & 0x1F) > 0).all()
        bits = bits + 0x400
        d2[..., 0] = bits & 0xFF
        d2[..., 1] = bits >> 8
        mats2[e] = (g, u, d2.reshape(D, -1))
    x = S.hidden(2, 6, D)
    G = S.gate_matrix(2, D, E)
    r1 = O.moe_layer(x, G, None, _experts_from(mats, 0, O), k)
    r2 = O.moe_layer(x, G, None, _experts_from(mats2, 0, O), k)
    assert np.array_equal(r2["out"], 2 * r1["out"])


def pin_equivariance(O):
    D, F_, E, k = 64, 32, 8, 3
    blobs = S.expert_blobs(3, E, D, F_, S.FMT_Q4)
    mats = {e: S.split_blob(blobs[e], D, F_, 1) for e in range(E)}
    x = S.hidden(3, 9, D)
    G = S.gate_matrix(3, D, E)
    b = S.zipf_bias(3, E)
    r = O.moe_layer(x, G, b, _experts_from(mats, 1, O), k)
    perm_t = np.random.default_rng(1).permutation(9)
    rp = O.moe_layer(x[perm_t], G, b, _experts_from(mats, 1, O), k)
    assert np.allclose(rp["out"], r["out"][perm_t], rtol=1e-13, atol=1e-15)
    pe = np.random.default_rng(2).permutation(E)          # new label i holds old expert pe[i]
    inv = np.argsort(pe)
    mats_p = {i: mats[int(pe[i])] for i in range(E)}
    rr = O.moe_layer(x, G[:, pe], b[pe], _experts_from(mats_p, 1, O), k)
    assert np.array_equal(np.sort(inv[r["ids"]], axis=1), rr["ids"])
    assert np.allclose(rr["out"], r["out"], rtol=1e-13, atol=1e-15)


def pin_down_combine(O):
    """The down-only operator agrees with the layer fed its own SwiGLU activations, and
    with one expert reduces to a matmul."""
    import torch
    D, F_, E, k = 64, 32, 8, 3
    blobs = S.expert_blobs(4, E, D, F_, S.FMT_Q4)
    mats = {e: S.split_blob(blobs[e], D, F_, 1) for e in range(E)}
    ex = _experts_from(mats, 1, O)
    x = S.hidden(4, 5, D)
    G = S.gate_matrix(4, D, E)
    r = O.moe_layer(x, G, None, ex, k)
    h = np.zeros((5 * k, F_))
    for i, e in enumerate(r["ids"].ravel()):
        Wg, Wu, _ = ex.weights(int(e))
        h[i] = O.swiglu(x[i // k].astype(np.float64), Wg, Wu)
    assert np.allclose(O.down_combine(h, r["ids"], r["w"], ex), r["out"], rtol=1e-13, atol=1e-15)
    rng = np.random.default_rng(15)
    Wd, rd = _exact_matrix(rng, F_, D, 1)
    hh = rng.standard_normal((6, F_))
    out = O.down_combine(hh, np.zeros((6, 1), np.int32), np.ones((6, 1)),
                         _experts_from({0: (None, None, rd)}, 1, O))
    assert np.allclose(out, (torch.from_numpy(hh) @ torch.from_numpy(Wd)).numpy(), rtol=1e-13, atol=1e-14)


def pin_rmsnorm(O):
    import torch
    rng = np.random.default_rng(16)
    o = rng.standard_normal((9, 2048)) * 3
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (2048,), eps=1e-6).numpy()
    got = O.rmsnorm(o, 1e-6)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)
    m = (o * o).mean(axis=1)
    assert np.allclose((got * got).mean(axis=1), m / (m + 1e-6), rtol=1e-13)


def pin_stack_zero_experts(O):
    """With all-zero expert blocks the stack is in_{l+1} = rmsnorm(in_l)."""
    D, F_, E, k = 64, 32, 8, 2
    zero = np.zeros((E, S.blob_layout(D, F_, 0)["stride"]), np.uint8)
    mats = {e: S.split_blob(zero[e], D, F_, 0) for e in range(E)}
    x0 = S.hidden(5, 4, D) * 3
    layers = [(S.gate_matrix(5, D, E, layer=l), S.zipf_bias(5, E, layer=l), _experts_from(mats, 0, O))
              for l in range(3)]
    res = O.stack(x0, layers, k)
    cur = x0.astype(np.float64)
    for l in range(3):
        assert np.array_equal(res[l]["out"], cur)
        cur = cur / np.sqrt((cur ** 2).mean(axis=1, keepdims=True) + 1e-6)


def pin_stack_live_experts(O):
    """Stacks of live layers against a torch float64 composition written out here:
    o_1 = x + MoE_1(x), then in_{l+1} = rms_norm(o_l) and o_{l+1} = in_{l+1} + MoE_{l+1}(in_{l+1}).

    Two stacks of three layers: one expert per layer with top-1 (MoE = that dense
    SwiGLU FFN), and three experts per layer all selected (k = E, so MoE = sum_e
    softmax(l)_e FFN_e with scipy's softmax).  Live experts make o_l differ from
    in_l, so normalising the wrong vector, dropping the residual, normalising
    before the first layer or skipping a norm all move the result."""
    import torch
    import torch.nn.functional as Fn
    from scipy.special import softmax
    rng = np.random.default_rng(17)
    D, F_ = 64, 96
    for E in (1, 3):
        layers, dense_layers = [], []
        for l in range(3):
            fmt = (l + E) % 2
            mats, dense = {}, []
            for e in range(E):
                Wg, rg = _exact_matrix(rng, D, F_, fmt)
                Wu, ru = _exact_matrix(rng, D, F_, fmt)
                Wd, rd = _exact_matrix(rng, F_, D, fmt)
                mats[e] = (rg, ru, rd)
                dense.append(tuple(torch.from_numpy(m) for m in (Wg, Wu, Wd)))
            G = (rng.standard_normal((D, E)) * 0.3).astype(np.float32)
            b = rng.standard_normal(E).astype(np.float32)
            layers.append((G, b, _experts_from(mats, fmt, O)))
            dense_layers.append((G, b, dense))
        x0 = (rng.standard_normal((5, D)) * 2.0).astype(np.float32)
        cur = torch.from_numpy(x0).double()
        ins, outs = [], []
        for l, (G, b, dense) in enumerate(dense_layers):
            if l > 0:
                cur = Fn.rms_norm(outs[-1], (D,), eps=1e-6)
            p = softmax(cur.numpy() @ G.astype(np.float64) + b.astype(np.float64), axis=1)
            mix = sum(torch.from_numpy(p[:, e:e + 1]) *
                      ((Fn.silu(cur @ Wg) * (cur @ Wu)) @ Wd)
                      for e, (Wg, Wu, Wd) in enumerate(dense))
            ins.append(cur)
            outs.append(cur + mix)
        res = O.stack(x0, layers, E)
        assert len(res) == 3
        for l in range(3):
            scale = float(outs[l].abs().max())
            assert np.allclose(res[l]["out"], outs[l].numpy(), rtol=1e-12, atol=1e-12 * scale), (E, l)
            assert np.allclose(res[l]["in"], ins[l].numpy(), rtol=1e-12, atol=1e-12), (E, l)
        # the layers are live: o_l is far from in_l, so the recurrences differ
        assert min(np.abs(r["out"] - r["in"]).max() for r in res) > 0.1


def pin_topk_gap(O):
    """The k-th minus (k+1)-th largest logit per row, against a Python sort of each
    row (exact ties give a gap of 0; k = E gives +inf)."""
    rng = np.random.default_rng(18)
    for trial in range(200):
        E = int(rng.integers(2, 12))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 5))
        l = rng.standard_normal((T, E)) if trial % 2 else rng.integers(-2, 3, (T, E)).astype(float)
        got = O.topk_gap(l, k)
        assert got.shape == (T,)
        for t in range(T):
            s = sorted(l[t].tolist(), reverse=True)
            want = math.inf if k == E else s[k - 1] - s[k]
            assert got[t] == want, (l[t], k, got[t], want)
    # a tie across the k-th / (k+1)-th boundary has no gap; a clear one has its size
    assert O.topk_gap(np.array([[3.0, 1.0, 1.0, 0.0]]), 2)[0] == 0.0
    assert O.topk_gap(np.array([[3.0, 1.0, 0.25, 0.0]]), 2)[0] == 0.75


# ---------------------------------------------------------------------------
# Attention-side primitives (input norm, Q/K/V projection, per-head Q/K norm,
# RoPE, KV append)
# ---------------------------------------------------------------------------

def _rope_complex(x, pos, theta):
    """RoPE as complex multiplication: z_i = x_i + j x_{i+hd/2} times e^{j pos theta^(-2i/hd)}."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    z = x[..., :half] + 1j * x[..., half:]
    freq = theta ** (-2.0 * np.arange(half) / x.shape[-1])
    rot = np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None, None] * freq[None, None, :])
    w = z * rot
    return np.concatenate([w.real, w.imag], axis=-1)


def pin_rope(O):
    """RoPE equals rotation of the complex pairs (x_i, x_{i+hd/2}); it preserves each
    pair's norm, is the identity at position 0, and q.k after RoPE depends only on the
    position difference."""
    rng = np.random.default_rng(19)
    x = rng.standard_normal((6, 3, 64))
    pos = np.array([0, 1, 7, 100, 4095, 8191])
    got = O.rope(x, pos, 1e6)
    assert np.allclose(got, _rope_complex(x, pos, 1e6), rtol=0, atol=1e-12)
    assert np.array_equal(got[0], x[0])
    half = 32
    pn = lambda a: a[..., :half] ** 2 + a[..., half:] ** 2      # noqa: E731
    assert np.allclose(pn(got), pn(x), rtol=1e-12, atol=1e-12)
    q, k = rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64))
    for m, n in ((5, 2), (900, 17), (3, 3)):
        a = (O.rope(q, [m], 1e4) * O.rope(k, [n], 1e4)).sum()
        b = (O.rope(q, [m - n], 1e4) * O.rope(k, [0], 1e4)).sum()
        assert abs(a - b) < 1e-9 * (1 + abs(a)), (m, n, a, b)


def pin_rmsnorm_gain(O):
    import torch
    rng = np.random.default_rng(20)
    x = rng.standard_normal((5, 4, 128)) * 2
    g = 1 + 0.1 * rng.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(g),
                                       eps=1e-6).numpy()
    assert np.allclose(O.rmsnorm_gain(x, g, 1e-6), ref, rtol=1e-13, atol=0)


def pin_attn_prep(O):
    """The whole primitive chain against a torch float64 composition written out here:
    rms_norm(x, gain) -> u W (exact block matrix; rows ordered q heads, k heads, v heads)
    -> per-head rms_norm with the q / k gains -> RoPE by complex multiplication; v is
    neither normalised nor rotated."""
    import torch
    import torch.nn.functional as Fn
    rng = np.random.default_rng(21)
    D, nq, nkv, hd = 96, 3, 2, 32
    for fmt in (O.Q8_0, O.Q4):
        W, raw = _exact_matrix(rng, D, (nq + 2 * nkv) * hd, fmt)
        x = rng.standard_normal((4, D)).astype(np.float32) * 3
        ga = (1 + 0.2 * rng.standard_normal(D)).astype(np.float32)
        gq = (1 + 0.2 * rng.standard_normal(hd)).astype(np.float32)
        gk = (1 + 0.2 * rng.standard_normal(hd)).astype(np.float32)
        pos = np.array([0, 3, 17, 250])
        r = O.attn_prep(x, raw, fmt, ga, gq, gk, pos, 1e6, nq, nkv, hd)
        t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))       # noqa: E731
        u = Fn.rms_norm(t(x), (D,), weight=t(ga), eps=1e-6)
        qkv = (u @ t(W)).numpy()
        q = qkv[:, :nq * hd].reshape(4, nq, hd)
        k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(4, nkv, hd)
        v = qkv[:, (nq + nkv) * hd:].reshape(4, nkv, hd)
        q = _rope_complex(Fn.rms_norm(t(q), (hd,), weight=t(gq), eps=1e-6).numpy(), pos, 1e6)
        k = _rope_complex(Fn.rms_norm(t(k), (hd,), weight=t(gk), eps=1e-6).numpy(), pos, 1e6)
        for name, ref in (("q", q), ("k", k), ("v", v)):
            assert np.allclose(r[name], ref, rtol=1e-11, atol=1e-11), (fmt, name)


def pin_kv_append(O):
    """Token t's k and v land at row pos[t] of the caches; no other row changes."""
    rng = np.random.default_rng(22)
    kc, vc = np.full((10, 2, 4), 7.0), np.full((10, 2, 4), -7.0)
    k, v = rng.standard_normal((3, 2, 4)), rng.standard_normal((3, 2, 4))
    pos = np.array([4, 0, 9])
    O.kv_append(kc, vc, k, v, pos)
    for t, p_ in enumerate(pos):
        assert np.array_equal(kc[p_], k[t]) and np.array_equal(vc[p_], v[t])
    rest = np.setdiff1d(np.arange(10), pos)
    assert (kc[rest] == 7.0).all() and (vc[rest] == -7.0).all()


ALL_PINS = [
    pin_page_expert_size, pin_fp16_decoder, pin_q8_0_exhaustive, pin_q4_exhaustive,
    pin_matrix_orientation, pin_encoder_roundtrip, pin_topk_bruteforce, pin_tie_break_zero_gate,
    pin_weights_closed_form, pin_full_selection_is_softmax, pin_router_logits, pin_grouping,
    pin_dense_reduction, pin_all_experts_mixture, pin_zero_input, pin_scalar_bruteforce,
    pin_linearity, pin_equivariance, pin_down_combine, pin_rmsnorm, pin_stack_zero_experts,
    pin_stack_live_experts, pin_topk_gap, pin_rope, pin_rmsnorm_gain, pin_attn_prep,
    pin_kv_append,
]


def failing_pins(O, pins=None):
    """Names of the pins that fail for oracle module ``O``."""
    failed = []
    for p in pins or ALL_PINS:
        try:
            p(O)
        except (AssertionError, ValueError, IndexError, TypeError) as e:  # a planted bug may crash
            failed.append(p.__name__)
            _ = e
    return failed


def rel_max_err(got, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float((ref * ref).mean()))
    return float(np.abs(np.asarray(got, dtype=np.float64) - ref).max()) / max(rms, 1e-300)
