"""Plant plausible mistakes in the CPU oracle and check that some pin catches each.

Every mutation is applied to the oracle module on the CPU only (monkeypatch),
then the whole pin suite runs against it; at least one pin must fail.
"""
import numpy as np
import pytest

import pins
from oracle import moe_oracle as O

_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}


def _decode_nibbles_swapped(raw, fmt):
    if fmt != O.Q4:
        return _orig["decode_rows"](raw, fmt)
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    rows, nb = raw.shape[0], raw.shape[1] // 18
    blk = raw.reshape(rows, nb, 18)
    d = O.fp16_bits_to_f64(blk[..., 0].astype(np.uint32) | (blk[..., 1].astype(np.uint32) << 8))
    q = np.empty((rows, nb, 32))
    q[..., 0::2] = blk[..., 2:] >> 4
    q[..., 1::2] = blk[..., 2:] & 15
    return (d[..., None] * (q - 8)).reshape(rows, nb * 32)


def _decode_no_offset(raw, fmt):
    v = _orig["decode_rows"](raw, fmt)
    if fmt != O.Q4:
        return v
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    rows, nb = raw.shape[0], raw.shape[1] // 18
    blk = raw.reshape(rows, nb, 18)
    d = O.fp16_bits_to_f64(blk[..., 0].astype(np.uint32) | (blk[..., 1].astype(np.uint32) << 8))
    return v + 8 * np.repeat(d, 32, axis=1).reshape(rows, nb * 32)


def _decode_unsigned_q8(raw, fmt):
    v = _orig["decode_rows"](raw, fmt)
    if fmt != O.Q8_0:
        return v
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    rows, nb = raw.shape[0], raw.shape[1] // 34
    blk = raw.reshape(rows, nb, 34)
    d = O.fp16_bits_to_f64(blk[..., 0].astype(np.uint32) | (blk[..., 1].astype(np.uint32) << 8))
    return (d[..., None] * blk[..., 2:].astype(np.float64)).reshape(rows, nb * 32)


def _fp16_bias_off(bits):
    return _orig["fp16_bits_to_f64"](bits) * 2.0


def _fp16_no_subnormal(bits):
    v = _orig["fp16_bits_to_f64"](bits)
    b = np.asarray(bits, dtype=np.uint32)
    return np.where(((b >> 10) & 0x1F) == 0, 0.0, v)


def _dequant_not_transposed(raw, fmt):
    v = O.decode_rows(raw, fmt)
    return v.reshape(v.shape[1], v.shape[0])


def _topk_high_index_ties(logits, k):
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.argsort(-logits[t][::-1], kind="stable")
        ids[t] = np.sort(E - 1 - order[:k])
    return ids


def _topk_unsorted(logits, k):
    ids = np.empty((logits.shape[0], k), dtype=np.int32)
    for t in range(logits.shape[0]):
        ids[t] = np.argsort(-logits[t], kind="stable")[:k]
    return ids


def _weights_not_renormalised(logits, ids):
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, ids.astype(np.int64), axis=1)


def _silu_is_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _swiglu_swapped(x, Wg, Wu):
    return O.silu(x @ Wu) * (x @ Wg)


def _combine_unweighted(y, w, residual=None):
    return _orig["combine"](y, np.ones_like(w), residual)


def _group_unstable(ids, E):
    off, rows = _orig["group"](ids, E)
    rows = rows.copy()
    for e in range(E):
        rows[off[e]:off[e + 1]] = rows[off[e]:off[e + 1]][::-1]
    return off, rows


def _rmsnorm_eps_outside(o, eps=1e-6):
    o = np.asarray(o, dtype=np.float64)
    return o / (np.sqrt((o * o).mean(axis=-1, keepdims=True)) + eps)


def _logits_no_bias(x, G, bias=None):
    return _orig["router_logits"](x, G, None)


def _expert_outputs_wrong_token(x, ids, experts):
    x = np.asarray(x, dtype=np.float64)
    T, k = ids.shape
    flat = ids.ravel()
    y = None
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        Wg, Wu, Wd = experts.weights(int(e))
        ye = O.swiglu(x[rows % T], Wg, Wu) @ Wd
        if y is None:
            y = np.zeros((T * k, ye.shape[1]))
        y[rows] = ye
    return y


def _expert_bytes_q4(D, F, fmt):
    return _orig["expert_bytes"](D, F, O.Q4)


def _stack_no_residual(x0, layers, k, eps=1e-6, on_layer=None):
    cur = np.asarray(x0, dtype=np.float64)
    res = []
    for l, (G, b, ex) in enumerate(layers):
        if l > 0:
            cur = O.rmsnorm(res[-1]["out"], eps)
        r = O.moe_layer(cur, G, b, ex, k, residual=False)
        res.append(r)
    return res


def _stack_normalises_input(x0, layers, k, eps=1e-6, on_layer=None):
    cur = np.asarray(x0, dtype=np.float64)
    res = []
    for l, (G, b, ex) in enumerate(layers):
        if l > 0:
            cur = O.rmsnorm(cur, eps)          # in_l instead of o_l
        r = O.moe_layer(cur, G, b, ex, k, residual=True)
        r["in"] = cur
        res.append(r)
    return res


def _gap_vacuous(logits, k):
    return np.full(np.asarray(logits).shape[0], np.inf)


def _gap_off_by_one(logits, k):
    T, E = logits.shape
    s = -np.sort(-logits, axis=1)
    if k + 1 >= E:
        return np.full(T, np.inf)
    return s[:, k] - s[:, k + 1]


def _rope_negative_angle(x, pos, theta):
    return _orig["rope"](x, -np.asarray(pos), theta)


def _rope_interleaved(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])
    inv = np.argsort(perm)
    return _orig["rope"](x[..., perm], pos, theta)[..., inv]


def _rope_half_frequency(x, pos, theta):
    return _orig["rope"](x, pos, theta ** 0.5)


def _attn_norm_over_all_heads(x, w_qkv_raw, fmt, attn_gain, q_gain, k_gain, pos, theta, n_q,
                              n_kv, head_dim, eps=1e-6):
    r = _orig["attn_prep"](x, w_qkv_raw, fmt, attn_gain, q_gain, k_gain, pos, theta, n_q, n_kv,
                           head_dim, eps)
    T = r["qkv"].shape[0]
    q = r["qkv"][:, :n_q * head_dim]
    q = O.rmsnorm(q, eps).reshape(T, n_q, head_dim) * np.asarray(q_gain, np.float64)
    r["q"] = O.rope(q, pos, theta)
    return r


def _attn_v_normalised(*a, **kw):
    r = _orig["attn_prep"](*a, **kw)
    r["v"] = O.rmsnorm(r["v"])
    return r


def _attn_k_not_rotated(x, w_qkv_raw, fmt, attn_gain, q_gain, k_gain, pos, theta, n_q, n_kv,
                        head_dim, eps=1e-6):
    r = _orig["attn_prep"](x, w_qkv_raw, fmt, attn_gain, q_gain, k_gain, pos, theta, n_q, n_kv,
                           head_dim, eps)
    T = r["qkv"].shape[0]
    k = r["qkv"][:, n_q * head_dim:(n_q + n_kv) * head_dim].reshape(T, n_kv, head_dim)
    r["k"] = O.rmsnorm_gain(k, k_gain, eps)
    return r


def _rmsnorm_gain_dropped(x, gain, eps=1e-6):
    return O.rmsnorm(x, eps)


def _kv_append_off_by_one(k_cache, v_cache, k, v, pos):
    _orig["kv_append"](k_cache, v_cache, k, v, (np.asarray(pos) + 1) % k_cache.shape[0])


MUTATIONS = {
    "q4 nibble order swapped": ("decode_rows", _decode_nibbles_swapped),
    "q4 missing -8": ("decode_rows", _decode_no_offset),
    "q8_0 read as unsigned": ("decode_rows", _decode_unsigned_q8),
    "fp16 exponent bias off by one": ("fp16_bits_to_f64", _fp16_bias_off),
    "fp16 subnormals flushed": ("fp16_bits_to_f64", _fp16_no_subnormal),
    "stored rows not transposed": ("dequant_matrix", _dequant_not_transposed),
    "ties to the higher index": ("select_topk", _topk_high_index_ties),
    "ids not in ascending order": ("select_topk", _topk_unsorted),
    "weights not renormalised": ("routing_weights", _weights_not_renormalised),
    "silu replaced by sigmoid": ("silu", _silu_is_sigmoid),
    "gate and up swapped": ("swiglu", _swiglu_swapped),
    "combine ignores weights": ("combine", _combine_unweighted),
    "grouping not stable": ("group", _group_unstable),
    "rmsnorm eps outside the root": ("rmsnorm", _rmsnorm_eps_outside),
    "router bias dropped": ("router_logits", _logits_no_bias),
    "expert fed the wrong token": ("expert_outputs", _expert_outputs_wrong_token),
    "expert size from the 4-bit format": ("expert_bytes", _expert_bytes_q4),
    "stack without residual": ("stack", _stack_no_residual),
    "stack normalises in_l instead of o_l": ("stack", _stack_normalises_input),
    "gap rule vacuous": ("topk_gap", _gap_vacuous),
    "gap taken one rank too low": ("topk_gap", _gap_off_by_one),
    "rope rotates the wrong way": ("rope", _rope_negative_angle),
    "rope pairs adjacent elements": ("rope", _rope_interleaved),
    "rope frequencies off": ("rope", _rope_half_frequency),
    "q normalised over all heads at once": ("attn_prep", _attn_norm_over_all_heads),
    "v normalised": ("attn_prep", _attn_v_normalised),
    "k not rotated": ("attn_prep", _attn_k_not_rotated),
    "norm gain dropped": ("rmsnorm_gain", _rmsnorm_gain_dropped),
    "kv append one row off": ("kv_append", _kv_append_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(O, attr, bad)
    failed = pins.failing_pins(O)
    assert failed, f"no pin caught: {name}"
