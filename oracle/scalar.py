"""Scalar-loop brute-force oracle for tiny inputs (pure Python floats).

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle.moe_oracle``).  It
shares no code with the vectorised oracle: fp16 scales are decoded with
``struct`` ('<e'), every dot product is a Python loop, top-k is a search over
all k-subsets, and grouping is a sort of (expert, flat index) pairs.  It exists
to check the vectorised oracle on tiny inputs, so it favours obviousness over
speed; keep inputs to a few thousand multiply-adds per output.
"""
from __future__ import annotations

import itertools
import math
import struct


def fp16(b0: int, b1: int) -> float:
    return struct.unpack("<e", bytes([b0, b1]))[0]


def block_values(block: bytes, fmt: int) -> list:
    """One block's 32 weights.  fmt 0 = Q8_0 (34 B), 1 = 4-bit (18 B)."""
    d = fp16(block[0], block[1])
    if fmt == 0:
        return [d * (b - 256 if b >= 128 else b) for b in block[2:34]]
    vals = []
    for b in block[2:18]:
        vals.append(d * ((b & 15) - 8))
        vals.append(d * ((b >> 4) - 8))
    return vals


def matrix(raw_rows, fmt: int) -> list:
    """Stored rows -> logical [in][out] list of lists."""
    bb = 34 if fmt == 0 else 18
    cols = []
    for row in raw_rows:
        row = bytes(row)
        vals = []
        for i in range(0, len(row), bb):
            vals.extend(block_values(row[i:i + bb], fmt))
        cols.append(vals)
    n_in = len(cols[0])
    return [[cols[o][i] for o in range(len(cols))] for i in range(n_in)]


def vecmat(v, M) -> list:
    return [sum(v[i] * M[i][o] for i in range(len(v))) for o in range(len(M[0]))]


def topk_bruteforce(l, k: int) -> list:
    """The k-subset S with every member beating every non-member on (value, lower index)."""
    E = len(l)

    def beats(a, b):
        return l[a] > l[b] or (l[a] == l[b] and a < b)

    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(beats(a, b) for a in S for b in rest):
            return list(S)
    raise AssertionError("no top-k subset")


def layer(x, G, bias, experts, fmt: int, k: int, residual: bool = False) -> dict:
    """``experts[e] = (gate_rows, up_rows, down_rows)`` raw bytes."""
    E = len(G[0])
    out, all_ids, all_w = [], [], []
    mats = {}
    for xt in x:
        l = vecmat(list(map(float, xt)), [list(map(float, r)) for r in G])
        if bias is not None:
            l = [a + float(b) for a, b in zip(l, bias)]
        ids = topk_bruteforce(l, k)
        # softmax restricted to the selected logits equals the renormalised full softmax
        m = max(l[e] for e in ids)
        ex = [math.exp(l[e] - m) for e in ids]
        s = sum(ex)
        w = [v / s for v in ex]
        acc = [float(v) if residual else 0.0 for v in xt]
        for wj, e in zip(w, ids):
            if e not in mats:
                mats[e] = tuple(matrix(r, fmt) for r in experts[e])
            Wg, Wu, Wd = mats[e]
            xv = list(map(float, xt))
            g = vecmat(xv, Wg)
            u = vecmat(xv, Wu)
            h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
            y = vecmat(h, Wd)
            acc = [a + wj * yi for a, yi in zip(acc, y)]
        out.append(acc)
        all_ids.append(ids)
        all_w.append(w)
    flat = [e for ids in all_ids for e in ids]
    pairs = sorted((e, i) for i, e in enumerate(flat))
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    return {"ids": all_ids, "w": all_w, "out": out, "offsets": offsets,
            "sorted_rows": [i for _, i in pairs]}
