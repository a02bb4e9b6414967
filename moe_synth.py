"""Seeded synthetic inputs for the routed MoE layer.

This module is the only code shared by the GPU path's tests/benchmark and the
CPU oracle.  It draws random inputs and encodes weights into the two block
formats; it holds none of the layer's arithmetic (no routing, no dequantised
products, no FFN, no combine).

Workloads follow the Qwen3-MoE geometry stated on the MER evidence page
(amalgafy.com/evidence, "Historical baseline environment" / Model: d_model 2048,
d_ff 768, 48 layers, 128 experts, learned top-8 routing) with synthetic values:

* hidden states x ~ N(0, 1), fp32;
* LinearGate matrix G ~ N(0, 0.02), fp32, shape [D][E] (logits = x @ G);
* per-expert logit bias b_e = -s * ln(r_e), r a seeded permutation of 1..E,
  i.e. the log of a Zipf(s) popularity (the normalising constant is dropped:
  softmax and top-k ignore a shift);
* expert matrices ~ N(0, 0.02), encoded block-wise along the reduction axis;
* attention-side inputs: Q/K/V projection rows ~ N(0, 0.02) block-encoded (q
  rows of every head, then k, then v), norm gains 1 + N(0, 0.1), distinct
  token positions drawn without replacement.

Every generator is numpy ``default_rng(SeedSequence([SEED, cfg, layer, role,
expert]))``.  Large weight arenas (hundreds of experts) are drawn on the GPU
with a seeded torch CUDA generator instead, because drawing ~10^10 normals on
the host takes far too long; those bytes are copied back for any host-side
check, so both sides always see identical bytes.

Block formats (the encoder here; decoding is the method's and lives elsewhere):

* Q8_0: 34 bytes per 32 weights: fp16 scale d (little-endian), then 32 int8 q.
  Encoder: d = fp16(max|w| / 127), q = clamp(rint(w / d), -127, 127); q = 0
  when d == 0.
* Q4 (4-bit): 18 bytes per 32 weights: fp16 scale d, then 16 bytes of nibbles,
  element 2i in the low nibble of byte i and 2i+1 in the high nibble, value
  d * (q - 8).  Encoder: d = fp16(max|w| / 7), q = clamp(rint(w / d) + 8, 0, 15);
  q = 8 when d == 0.

A weight matrix with logical shape [in][out] is stored as ``out`` rows of
``in / 32`` consecutive blocks (row n holds output column n).  One expert is one
contiguous blob: gate rows, then up rows, then down rows.
"""
from __future__ import annotations

import numpy as np

SEED = 0x4D4F45  # "MOE"

ROLE_X, ROLE_G, ROLE_ZIPF, ROLE_WG, ROLE_WU, ROLE_WD, ROLE_H, ROLE_REDRAW = range(8)
ROLE_WQKV, ROLE_GAIN, ROLE_POS = 8, 9, 10

FMT_Q8_0 = 0
FMT_Q4 = 1
BLOCK = 32
BLOCK_BYTES = {FMT_Q8_0: 34, FMT_Q4: 18}
PAGE = 4096


def generator(cfg: int, layer: int, role: int, expert: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED, cfg, layer, role, expert]))


def hidden(cfg: int, T: int, D: int, layer: int = 0) -> np.ndarray:
    """x ~ N(0, 1), fp32, [T][D]."""
    return generator(cfg, layer, ROLE_X).standard_normal((T, D), dtype=np.float32)


def redraw_row(cfg: int, row: int, attempt: int, D: int, layer: int = 0) -> np.ndarray:
    """A fresh N(0, 1) row for token ``row``, from its own sub-stream."""
    g = np.random.default_rng(np.random.SeedSequence([SEED, cfg, layer, ROLE_REDRAW, row, attempt]))
    return g.standard_normal(D, dtype=np.float32)


def redraw_until(x: np.ndarray, cfg: int, accept, layer: int = 0, max_attempts: int = 64):
    """Redraw rows of ``x`` (in place) until ``accept(x) -> bool[T]`` holds for all.

    ``accept`` is supplied by the caller; this module does not know what it
    computes.  Returns the per-row redraw counts.
    """
    T, D = x.shape
    counts = np.zeros(T, dtype=np.int64)
    ok = np.asarray(accept(x), dtype=bool)
    while not ok.all():
        bad = np.nonzero(~ok)[0]
        for r in bad:
            counts[r] += 1
            if counts[r] > max_attempts:
                raise RuntimeError(f"row {r}: no acceptable draw in {max_attempts} attempts")
            x[r] = redraw_row(cfg, int(r), int(counts[r]), D, layer)
        ok = np.asarray(accept(x), dtype=bool)
    return counts


def gate_matrix(cfg: int, D: int, E: int, layer: int = 0, std: float = 0.02) -> np.ndarray:
    """LinearGate weights, fp32 [D][E], N(0, std)."""
    g = generator(cfg, layer, ROLE_G)
    return (g.standard_normal((D, E), dtype=np.float32) * np.float32(std)).astype(np.float32)


def zipf_bias(cfg: int, E: int, s: float = 1.1, layer: int = 0) -> np.ndarray:
    """Per-expert logit bias, fp32 [E]: b_e = -s * ln(r_e), r a permutation of 1..E."""
    r = generator(cfg, layer, ROLE_ZIPF).permutation(E) + 1
    return (-s * np.log(r.astype(np.float64))).astype(np.float32)


def normal_rows(cfg: int, layer: int, role: int, expert: int, rows: int, cols: int,
                std: float = 0.02) -> np.ndarray:
    g = generator(cfg, layer, role, expert)
    return (g.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)).astype(np.float32)


# ----------------------------------------------------------------------------
# Block encoders (host, numpy)
# ----------------------------------------------------------------------------

def _scales_fp16(amax: np.ndarray, qmax: float) -> np.ndarray:
    return (amax / np.float32(qmax)).astype(np.float32).astype(np.float16)


def quantize_q8_0(w: np.ndarray) -> np.ndarray:
    """Encode rows of fp32 ``w`` [rows][n_in] (n_in % 32 == 0) to Q8_0 bytes."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, n_in = w.shape
    assert n_in % BLOCK == 0
    b = w.reshape(rows, n_in // BLOCK, BLOCK)
    d16 = _scales_fp16(np.abs(b).max(axis=2), 127.0)
    d = d16.astype(np.float32)
    safe = np.where(d > 0, d, np.float32(1))
    q = np.clip(np.rint(b / safe[..., None]), -127, 127)
    q = np.where(d[..., None] > 0, q, 0).astype(np.int8)
    out = np.empty((rows, n_in // BLOCK, 34), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(rows, n_in // BLOCK, 2)
    out[..., 2:34] = q.view(np.uint8)
    return out.reshape(rows, -1)


def quantize_q4(w: np.ndarray) -> np.ndarray:
    """Encode rows of fp32 ``w`` [rows][n_in] to the 4-bit block format."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, n_in = w.shape
    assert n_in % BLOCK == 0
    b = w.reshape(rows, n_in // BLOCK, BLOCK)
    d16 = _scales_fp16(np.abs(b).max(axis=2), 7.0)
    d = d16.astype(np.float32)
    safe = np.where(d > 0, d, np.float32(1))
    q = np.clip(np.rint(b / safe[..., None]) + 8, 0, 15)
    q = np.where(d[..., None] > 0, q, 8).astype(np.uint8)
    out = np.empty((rows, n_in // BLOCK, 18), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(rows, n_in // BLOCK, 2)
    out[..., 2:18] = q[..., 0::2] | (q[..., 1::2] << 4)
    return out.reshape(rows, -1)


def quantize(w: np.ndarray, fmt: int) -> np.ndarray:
    return quantize_q8_0(w) if fmt == FMT_Q8_0 else quantize_q4(w)


def matrix_bytes(rows: int, n_in: int, fmt: int) -> int:
    return rows * (n_in // BLOCK) * BLOCK_BYTES[fmt]


def blob_layout(D: int, F: int, fmt: int) -> dict:
    """Byte offsets of gate/up/down inside one expert blob, and the page-aligned stride."""
    g = matrix_bytes(F, D, fmt)
    dn = matrix_bytes(D, F, fmt)
    size = 2 * g + dn
    stride = (size + PAGE - 1) // PAGE * PAGE
    return {"gate": 0, "up": g, "down": 2 * g, "size": size, "stride": stride,
            "gate_bytes": g, "down_bytes": dn}


def expert_blobs(cfg: int, E: int, D: int, F: int, fmt: int, layer: int = 0,
                 std: float = 0.02) -> np.ndarray:
    """Host-drawn experts of one layer: uint8 [E][stride] (small geometries only)."""
    lay = blob_layout(D, F, fmt)
    out = np.zeros((E, lay["stride"]), dtype=np.uint8)
    for e in range(E):
        wg = normal_rows(cfg, layer, ROLE_WG, e, F, D, std)
        wu = normal_rows(cfg, layer, ROLE_WU, e, F, D, std)
        wd = normal_rows(cfg, layer, ROLE_WD, e, D, F, std)
        out[e, lay["gate"]:lay["up"]] = quantize(wg, fmt).ravel()
        out[e, lay["up"]:lay["down"]] = quantize(wu, fmt).ravel()
        out[e, lay["down"]:lay["size"]] = quantize(wd, fmt).ravel()
    return out


def split_blob(blob: np.ndarray, D: int, F: int, fmt: int):
    """(gate, up, down) byte matrices of one expert blob, each [rows][row_bytes]."""
    lay = blob_layout(D, F, fmt)
    bb = BLOCK_BYTES[fmt]
    gate = blob[lay["gate"]:lay["up"]].reshape(F, D // BLOCK * bb)
    up = blob[lay["up"]:lay["down"]].reshape(F, D // BLOCK * bb)
    down = blob[lay["down"]:lay["size"]].reshape(D, F // BLOCK * bb)
    return gate, up, down


# ----------------------------------------------------------------------------
# Device-drawn arenas (large geometries)
# ----------------------------------------------------------------------------

def _torch_quantize(w, fmt: int):
    """Same encoder as :func:`quantize`, on torch tensors (any device)."""
    import torch
    rows, n_in = w.shape
    nb = n_in // BLOCK
    b = w.reshape(rows, nb, BLOCK)
    qmax = 127.0 if fmt == FMT_Q8_0 else 7.0
    d16 = (b.abs().amax(dim=2) / qmax).to(torch.float16)
    d = d16.to(torch.float32)
    safe = torch.where(d > 0, d, torch.ones_like(d))
    r = torch.round(b / safe[..., None])  # round half to even, like numpy.rint
    bb = BLOCK_BYTES[fmt]
    out = torch.empty((rows, nb, bb), dtype=torch.uint8, device=w.device)
    out[..., 0:2] = d16.view(torch.uint8).reshape(rows, nb, 2)
    if fmt == FMT_Q8_0:
        q = torch.where(d[..., None] > 0, r.clamp(-127, 127), torch.zeros_like(r)).to(torch.int8)
        out[..., 2:34] = q.view(torch.uint8)
    else:
        q = torch.where(d[..., None] > 0, (r + 8).clamp(0, 15), torch.full_like(r, 8)).to(torch.uint8)
        out[..., 2:18] = q[..., 0::2] | (q[..., 1::2] << 4)
    return out.reshape(rows, nb * bb)


def device_arena(cfg: int, layers: int, E: int, D: int, F: int, fmt: int, device,
                 std: float = 0.02, which=("gate", "up", "down")):
    """Experts for ``layers`` layers drawn on ``device``: uint8 tensor [layers][E][stride].

    Each (layer, expert, matrix) is drawn from a torch generator seeded from
    (SEED, cfg, layer, role, expert).  Matrices not named in ``which`` are
    left zero-filled (e.g. a down-projection-only workload).
    """
    import torch
    lay = blob_layout(D, F, fmt)
    arena = torch.zeros((layers, E, lay["stride"]), dtype=torch.uint8, device=device)
    gen = torch.Generator(device=device)
    parts = (("gate", ROLE_WG, F, D), ("up", ROLE_WU, F, D), ("down", ROLE_WD, D, F))
    for l in range(layers):
        for name, role, rows, n_in in parts:
            if name not in which:
                continue
            off = lay[name]
            nbytes = matrix_bytes(rows, n_in, fmt)
            # one draw per (layer, role) covering all experts keeps this fast;
            # the seed still names (cfg, layer, role).
            seed = int(np.random.SeedSequence([SEED, cfg, l, role]).generate_state(1, np.uint64)[0] >> 1)
            gen.manual_seed(seed)
            w = torch.randn((E * rows, n_in), generator=gen, device=device, dtype=torch.float32) * std
            q = _torch_quantize(w, fmt).reshape(E, nbytes)
            arena[l, :, off:off + nbytes] = q
            del w, q
    return arena


# ----------------------------------------------------------------------------
# Attention-side inputs (input / per-head norm gains, Q/K/V projection rows)
# ----------------------------------------------------------------------------

def qkv_rows(n_q: int, n_kv: int, head_dim: int) -> int:
    return (n_q + 2 * n_kv) * head_dim


def attn_gain(cfg: int, n: int, which: int, layer: int = 0, std: float = 0.1) -> np.ndarray:
    """A norm gain vector, fp32 [n]: 1 + N(0, std) (which: 0 input, 1 q, 2 k)."""
    g = generator(cfg, layer, ROLE_GAIN, which)
    return (1.0 + g.standard_normal(n, dtype=np.float32) * np.float32(std)).astype(np.float32)


def qkv_weights(cfg: int, D: int, n_q: int, n_kv: int, head_dim: int, fmt: int, layer: int = 0,
                std: float = 0.02) -> np.ndarray:
    """Host-drawn Q/K/V projection: uint8 [(n_q + 2 n_kv) * head_dim][D/32 * block bytes]
    (q rows of every head, then k, then v), N(0, std) weights block-encoded."""
    N = qkv_rows(n_q, n_kv, head_dim)
    return quantize(normal_rows(cfg, layer, ROLE_WQKV, 0, N, D, std), fmt)


def device_qkv_arena(cfg: int, layers: int, D: int, n_q: int, n_kv: int, head_dim: int, fmt: int,
                     device, std: float = 0.02):
    """Q/K/V projections of several layers drawn on ``device``: uint8 [layers][N][row bytes]."""
    import torch
    N = qkv_rows(n_q, n_kv, head_dim)
    rb = D // BLOCK * BLOCK_BYTES[fmt]
    arena = torch.empty((layers, N, rb), dtype=torch.uint8, device=device)
    gen = torch.Generator(device=device)
    for l in range(layers):
        seed = int(np.random.SeedSequence([SEED, cfg, l, ROLE_WQKV]).generate_state(1, np.uint64)[0] >> 1)
        gen.manual_seed(seed)
        w = torch.randn((N, D), generator=gen, device=device, dtype=torch.float32) * std
        arena[l] = _torch_quantize(w, fmt)
        del w
    return arena


def positions(cfg: int, T: int, max_pos: int, layer: int = 0) -> np.ndarray:
    """Distinct token positions in [0, max_pos), int32 [T]."""
    return generator(cfg, layer, ROLE_POS).choice(max_pos, size=T, replace=False).astype(np.int32)
