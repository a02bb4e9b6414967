"""fp64 CPU oracle of the routed MoE layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
and its Python binding never import, call or link it, and it shares no code
with them: it decodes the block formats, routes, groups and runs the experts
with its own numpy code in float64.

What it computes (the routed MoE layer that MER's warm path runs as
"router -> resident expert -> combine", technical-overview page, "Execution
architecture", warm target path; geometry from the evidence page, "Historical
baseline environment", Model card: d_model 2048, d_ff 768, 128 experts per
layer, learned top-8 selection by a LinearGate router):

1. logits  l = x G + b                      (LinearGate router, fp64)
2. top-k   the k experts with the largest l, lower index first on ties,
           reported in ascending expert id
3. weights p = softmax(l) over all E experts, then w_j = p_{id_j} / sum_j p_{id_j}
4. grouping  counts per expert, exclusive scan, stable scatter of the flat
           (token, slot) index t*k + j, token-ascending inside each expert
5. expert  y = (silu(x W_gate) * (x W_up)) W_down, silu(z) = z / (1 + e^-z)
           (SwiGLU as defined by Shazeer, "GLU Variants Improve Transformer")
6. combine out_t = sum_j w_{t,j} y_{t,j}  (+ x_t with a residual)
7. stack   o_l = in_l + MoE_l(in_l), in_{l+1} = o_l / sqrt(mean(o_l^2) + eps)
8. attention-side primitives of the warm path: input RMSNorm with gain, Q/K/V
   projection, per-head Q/K RMSNorm, RoPE, KV append

Block formats (weights are "native Q8_0", evidence page, GPU-native foundation
card; "Q4 expert execution", technical-overview page, Execution architecture):
Q8_0 = fp16 scale d (little-endian) + 32 int8 q, w = d q; Q4 = fp16 scale d +
16 bytes of nibbles (element 2i low nibble of byte i, 2i+1 high nibble),
w = d (q - 8).  A logical [in][out] matrix is stored as ``out`` rows of
``in/32`` blocks.  Every product d*q is exact in float64.

Readings where the pages are silent are listed with the design notes of this
repository; each function below names the step it implements.
"""
from __future__ import annotations

import numpy as np

Q8_0 = 0
Q4 = 1
QK = 32                       # weights per block
Q8_0_BYTES = 2 + QK           # fp16 scale + 32 int8
Q4_BYTES = 2 + QK // 2        # fp16 scale + 16 bytes of nibbles


def block_bytes(fmt: int) -> int:
    if fmt == Q8_0:
        return Q8_0_BYTES
    if fmt == Q4:
        return Q4_BYTES
    raise ValueError(f"unknown block format {fmt}")


def expert_bytes(D: int, F: int, fmt: int) -> int:
    """Bytes of one expert (gate F x D, up F x D, down D x F), unpadded."""
    return (2 * F * (D // QK) + D * (F // QK)) * block_bytes(fmt)


# ---------------------------------------------------------------------------
# 1. Block decoding
# ---------------------------------------------------------------------------

def fp16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64, by sign/exponent/mantissa fields.

    Subnormals are honoured; exponent 31 gives inf/nan.
    """
    b = np.asarray(bits, dtype=np.uint32)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    ex = ((b >> 10) & 0x1F).astype(np.int64)
    man = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1024.0 + man, (ex - 25).astype(np.int32))
    sub = np.ldexp(man, -24)
    val = np.where(ex == 0, sub, normal)
    val = np.where(ex == 31, np.where(man == 0, np.inf, np.nan), val)
    return sign * val


def decode_rows(raw: np.ndarray, fmt: int) -> np.ndarray:
    """Stored rows of blocks, uint8 [rows][nb * block_bytes] -> float64 [rows][nb * 32]."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    bb = block_bytes(fmt)
    rows = raw.shape[0]
    assert raw.shape[1] % bb == 0
    nb = raw.shape[1] // bb
    blk = raw.reshape(rows, nb, bb)
    d = fp16_bits_to_f64(blk[..., 0].astype(np.uint32) | (blk[..., 1].astype(np.uint32) << 8))
    if fmt == Q8_0:
        q = blk[..., 2:].view(np.int8).astype(np.float64)            # two's complement
    else:
        nib = blk[..., 2:]
        q = np.empty((rows, nb, QK), dtype=np.float64)
        q[..., 0::2] = nib & 0x0F                                   # element 2i: low nibble
        q[..., 1::2] = nib >> 4                                     # element 2i+1: high nibble
        q -= 8.0
    return (d[..., None] * q).reshape(rows, nb * QK)


def dequant_matrix(raw: np.ndarray, fmt: int) -> np.ndarray:
    """Logical [in][out] float64 matrix from ``out`` stored rows of blocks."""
    return decode_rows(raw, fmt).T


# ---------------------------------------------------------------------------
# 2-3. Router: LinearGate logits, top-k with lower-index tie-break, weights
# ---------------------------------------------------------------------------

def router_logits(x, G, bias=None) -> np.ndarray:
    """l = x G (+ b), float64 [T][E]."""
    l = np.asarray(x, dtype=np.float64) @ np.asarray(G, dtype=np.float64)
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest logits per row, ties to the lower index, ascending ids."""
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # order by (-l_e, e): a stable sort of -l keeps equal logits in index order
        order = np.argsort(-logits[t], kind="stable")
        ids[t] = np.sort(order[:k])
    return ids


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """l_(k) - l_(k+1) per row (k-th minus (k+1)-th largest); +inf when k == E."""
    T, E = logits.shape
    if k >= E:
        return np.full(T, np.inf)
    s = -np.sort(-logits, axis=1)
    return s[:, k - 1] - s[:, k]


def routing_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over all E logits, then renormalise the selected k to sum 1."""
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x, G, bias, k: int):
    l = router_logits(x, G, bias)
    ids = select_topk(l, k)
    return ids, routing_weights(l, ids), l


# ---------------------------------------------------------------------------
# 4. Grouping: histogram, exclusive scan, stable scatter
# ---------------------------------------------------------------------------

def group(ids: np.ndarray, E: int):
    """(expert_offsets [E+1], sorted_rows [T*k]) for flat index t*k + j."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    rows = np.empty(flat.size, dtype=np.int64)
    for i, e in enumerate(flat):          # visiting i in order keeps it stable
        rows[cursor[e]] = i
        cursor[e] += 1
    return offsets.astype(np.int32), rows.astype(np.int32)


# ---------------------------------------------------------------------------
# 5-6. Expert SwiGLU FFN and weighted combine
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray) -> np.ndarray:
    """h = silu(x Wg) * (x Wu), float64."""
    return silu(x @ Wg) * (x @ Wu)


class Experts:
    """One layer's experts as raw blocks, decoded lazily and cached.

    ``fetch(e) -> (gate_raw, up_raw, down_raw)``; each raw matrix is uint8
    [rows][row_bytes] (gate/up: F rows of D/32 blocks, down: D rows of F/32).
    """

    def __init__(self, fetch, fmt: int):
        self.fetch = fetch
        self.fmt = fmt
        self._cache = {}

    def weights(self, e: int):
        if e not in self._cache:
            g, u, d = self.fetch(e)
            self._cache[e] = tuple(None if r is None else dequant_matrix(r, self.fmt)
                                   for r in (g, u, d))
        return self._cache[e]


def expert_outputs(x: np.ndarray, ids: np.ndarray, experts: Experts) -> np.ndarray:
    """y [T*k][D]: y[t*k+j] = FFN_{ids[t,j]}(x_t), expert by expert."""
    x = np.asarray(x, dtype=np.float64)
    T, k = ids.shape
    flat = ids.ravel()
    y = None
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        Wg, Wu, Wd = experts.weights(int(e))
        ye = swiglu(x[rows // k], Wg, Wu) @ Wd
        if y is None:
            y = np.zeros((T * k, ye.shape[1]))
        y[rows] = ye
    return y


def combine(y: np.ndarray, w: np.ndarray, residual=None) -> np.ndarray:
    """out_t = sum_j w_{t,j} y_{t*k+j} (+ residual_t)."""
    T, k = w.shape
    out = (np.asarray(w, dtype=np.float64)[:, :, None] * y.reshape(T, k, -1)).sum(axis=1)
    if residual is not None:
        out = out + np.asarray(residual, dtype=np.float64)
    return out


def moe_layer(x, G, bias, experts: Experts, k: int, residual: bool = False) -> dict:
    """Router -> grouping -> expert FFNs -> combine for one layer."""
    ids, w, l = route(x, G, bias, k)
    offsets, rows = group(ids, np.asarray(G).shape[1])
    y = expert_outputs(x, ids, experts)
    out = combine(y, w, np.asarray(x, dtype=np.float64) if residual else None)
    return {"ids": ids, "w": w, "logits": l, "offsets": offsets, "sorted_rows": rows,
            "y": y, "out": out}


def down_combine(h, ids: np.ndarray, w: np.ndarray, experts: Experts) -> np.ndarray:
    """Down projection of routed activations plus combine.

    ``h`` is [T*k][F] in flat (t, j) order; out_t = sum_j w_{t,j} (h_{t*k+j} W_down_{ids[t,j]}).
    """
    h = np.asarray(h, dtype=np.float64)
    T, k = ids.shape
    flat = ids.ravel()
    y = None
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        Wd = experts.weights(int(e))[2]
        ye = h[rows] @ Wd
        if y is None:
            y = np.zeros((T * k, ye.shape[1]))
        y[rows] = ye
    return combine(y, w)


# ---------------------------------------------------------------------------
# 7. Inter-layer RMSNorm and the layer stack
# ---------------------------------------------------------------------------

def rmsnorm(o, eps: float = 1e-6) -> np.ndarray:
    """o / sqrt(mean_D(o^2) + eps), unit gain."""
    o = np.asarray(o, dtype=np.float64)
    return o / np.sqrt((o * o).mean(axis=-1, keepdims=True) + eps)


def stack(x0, layers, k: int, eps: float = 1e-6, on_layer=None) -> list:
    """o_l = in_l + MoE_l(in_l); in_{l+1} = rmsnorm(o_l).

    ``layers`` yields (G, bias, Experts) per layer.  Returns the per-layer
    results of :func:`moe_layer` (``out`` is o_l, ``in`` is in_l).
    """
    cur = np.asarray(x0, dtype=np.float64)
    res = []
    for l, (G, b, ex) in enumerate(layers):
        if l > 0:
            cur = rmsnorm(res[-1]["out"], eps)
        r = moe_layer(cur, G, b, ex, k, residual=True)
        r["in"] = cur
        if on_layer is not None:
            on_layer(l, r)
        res.append(r)
    return res


# ---------------------------------------------------------------------------
# 8. Attention-side primitives of the warm decode path (technical-overview page,
#    "Validated GPU foundation": RMSNorm, grouped per-head Q/K normalization,
#    Q/K/V projections, RoPE, request-local F32 KV append).  Attention itself
#    (scores, softmax, value aggregation, output projection) is not here: the
#    same page lists it as still being integrated.
# ---------------------------------------------------------------------------

def rmsnorm_gain(x, gain, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    return rmsnorm(x, eps) * np.asarray(gain, dtype=np.float64)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing: for i < hd/2 the pair
    (x_i, x_{i+hd/2}) is rotated by the angle pos * theta^(-2i/hd).

    ``x`` [T][H][hd], ``pos`` [T] (integers)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]      # [T][half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def attn_prep(x, w_qkv_raw, fmt: int, attn_gain, q_gain, k_gain, pos, theta: float,
              n_q: int, n_kv: int, head_dim: int, eps: float = 1e-6) -> dict:
    """One token block through the attention-side primitives:
    u = rmsnorm(x) * attn_gain; [q | k | v] = u W_qkv (rows of blocks: n_q heads
    of q, then n_kv of k, then n_kv of v, head_dim rows each); per-head
    RMSNorm of q and k with the shared gains q_gain / k_gain [head_dim]; RoPE
    of q and k at each token's position.  Returns q [T][n_q][hd], and the k and
    v rows [T][n_kv][hd] that the KV append writes at row pos[t] of the cache."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    u = rmsnorm_gain(x, attn_gain, eps)
    qkv = u @ dequant_matrix(w_qkv_raw, fmt)
    nq, nk = n_q * head_dim, n_kv * head_dim
    q = qkv[:, :nq].reshape(T, n_q, head_dim)
    k = qkv[:, nq:nq + nk].reshape(T, n_kv, head_dim)
    v = qkv[:, nq + nk:nq + 2 * nk].reshape(T, n_kv, head_dim)
    q = rope(rmsnorm_gain(q, q_gain, eps), pos, theta)
    k = rope(rmsnorm_gain(k, k_gain, eps), pos, theta)
    return {"u": u, "qkv": qkv, "q": q, "k": k, "v": v}


def kv_append(k_cache, v_cache, k, v, pos) -> None:
    """Write token t's k and v rows at row pos[t] of the caches ([max_pos][n_kv][hd])."""
    for t, p in enumerate(np.asarray(pos)):
        k_cache[int(p)] = k[t]
        v_cache[int(p)] = v[t]
