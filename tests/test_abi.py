"""C ABI on the CPU: the library loads, exports every declared call, and rejects bad
arguments on the host before any HIP call (so no GPU is needed here)."""
import ctypes
import os
import re

import pytest

import mixture_experts_routed_lineargate_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH), reason="library not built")

FAKE = 0x10000  # a well-aligned non-NULL address that is never dereferenced on error paths


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(M.EXPORTS)


def test_every_declared_symbol_is_exported():
    L = M.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert M.abi_version() == 1


def test_status_strings():
    for s in range(11):
        assert M.status_str(s) != "unknown status"
    assert M.status_str(0) == "ok"
    assert M.status_str(11) == "unknown status"


def test_workspace_bytes():
    L = M.lib()
    assert L.moe_workspace_bytes(0, 2048, 768, 128, 8, 0, 0) == 0
    n1 = L.moe_workspace_bytes(1, 2048, 768, 128, 8, 0, 0)
    n32 = L.moe_workspace_bytes(32, 2048, 768, 128, 8, 1, 0)
    n1024 = L.moe_workspace_bytes(1024, 2048, 768, 128, 8, 1, 0)
    assert 0 < n1 < n32 < n1024
    # h and y buffers for every routed row must fit
    assert n1024 >= 1024 * 8 * (768 + 2048) * 4
    assert L.moe_workspace_bytes(16, 256, 128, 16, 2, 0, M.F_PRENORM) > \
        L.moe_workspace_bytes(16, 256, 128, 16, 2, 0, 0)


def _experts(**kw):
    base = dict(num_experts=128, d_model=2048, d_ff=768, format=0, w_gate=FAKE,
                gate_stride=5013504, w_up=FAKE, up_stride=5013504, w_down=FAKE,
                down_stride=5013504)
    base.update(kw)
    return M.moe_experts(**base)


def _layer(ex, T=4, k=8, flags=0, x=FAKE, gate=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return M.lib().moe_layer(x, gate, None, ctypes.byref(ex), T, k, flags, out, None, None, None,
                             None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(format=7), 4),
    (dict(d_model=2000), 2),
    (dict(d_ff=100), 2),
    (dict(num_experts=0), 2),
    (dict(num_experts=2048), 6),
    (dict(w_gate=None), 1),
    (dict(w_down=None), 1),
    (dict(w_up=FAKE + 1), 3),
    (dict(gate_stride=5013505), 3),
])
def test_layer_rejects_bad_experts(kw, status):
    assert _layer(_experts(**kw)) == status


def test_layer_rejects_bad_arguments():
    ex = _experts()
    assert _layer(ex, k=0) == 2
    assert _layer(ex, k=129) == 2
    assert _layer(ex, k=33) == 6
    assert _layer(ex, T=-1) == 2
    assert _layer(ex, x=None) == 1
    assert _layer(ex, out=None) == 1
    assert _layer(ex, x=FAKE + 2) == 3
    assert _layer(ex, ws=None) == 5
    assert _layer(ex, ws_bytes=1000) == 5
    assert _layer(ex, T=0) == 0          # empty input: nothing enqueued
    assert _layer(ex, out=FAKE + 4 * 4 * 2048 - 4) == M.MOE_E_OVERLAP   # last x row meets out


def test_route_group_combine_validation():
    L = M.lib()
    assert L.moe_route(FAKE, 1, 2048, FAKE, None, 128, 8, FAKE, FAKE, FAKE, 10, None) == 5
    assert L.moe_route(FAKE, 1, 2047, FAKE, None, 128, 8, FAKE, FAKE, FAKE, 1 << 40, None) == 2
    assert L.moe_route(None, 1, 2048, FAKE, None, 128, 8, FAKE, FAKE, FAKE, 1 << 40, None) == 1
    assert L.moe_route(FAKE, 0, 2048, FAKE, None, 128, 8, FAKE, FAKE, FAKE, 0, None) == 0
    assert L.moe_group(FAKE, 4, 9, 8, FAKE, FAKE, None, 0, None) == 2
    assert L.moe_group(None, 4, 2, 8, FAKE, FAKE, None, 0, None) == 1
    assert L.moe_group(FAKE, 0, 2, 8, FAKE, FAKE, None, 0, None) == 0
    assert L.moe_combine(FAKE, FAKE, 4, 0, 2048, None, FAKE, None) == 2
    assert L.moe_combine(FAKE, None, 4, 8, 2048, None, FAKE, None) == 1
    far = FAKE + (1 << 32)
    assert L.moe_combine(FAKE, far, 4, 8, 2048, None, FAKE + 4096, None) == M.MOE_E_OVERLAP
    assert L.moe_combine(FAKE, far, 4, 8, 2048, far + (1 << 20) + 4, far + (1 << 20), None) == \
        M.MOE_E_OVERLAP                                                   # shifted residual
    assert L.moe_rmsnorm(FAKE, 4, 2048, -1.0, FAKE, None) == 2
    assert L.moe_rmsnorm(FAKE, 0, 2048, 1e-6, FAKE, None) == 0


def test_expert_ffn_validation():
    L = M.lib()
    ex = _experts()
    args = lambda stage=0, y=FAKE, out=None, w=FAKE, ws=FAKE: L.moe_expert_ffn(  # noqa: E731
        FAKE, stage, ctypes.byref(ex), FAKE, w, FAKE, FAKE, 4, 8, y, out, 0, ws, 1 << 40, None)
    assert args(stage=5) == 4
    assert args(y=None, out=None) == 1
    assert args(y=None, out=FAKE, w=None) == 1
    assert args(ws=None) == 5
    assert args(y=FAKE + 4096) == M.MOE_E_OVERLAP                        # y inside x
    assert args(y=None, out=FAKE + 4 * 2048 * 4 - 4) == M.MOE_E_OVERLAP  # out meets x
    down_only = _experts(w_gate=None, w_up=None)
    assert L.moe_expert_ffn(FAKE, 0, ctypes.byref(down_only), FAKE, FAKE, FAKE, FAKE, 4, 8, FAKE,
                            None, 0, FAKE, 1 << 40, None) == 1


def test_layer_noalloc_validation():
    """The allocation-free layer rejects bad arguments, and shapes whose workspace
    exceeds its 8 MiB static array, on the host before any HIP call."""
    L = M.lib()
    ex = _experts()

    def call(T=4, k=8, x=FAKE, out=FAKE, e=ex):
        return L.moe_layer_noalloc(x, FAKE, None, ctypes.byref(e), T, k, 0, out, None, None,
                                   None, None, None)
    assert call(T=0) == 0
    assert call(x=None) == 1
    assert call(out=None) == 1
    assert call(k=0) == 2
    assert call(x=FAKE + 2) == 3
    assert call(e=_experts(format=9)) == 4
    assert call(T=64) == 6                      # > 8 MiB of workspace at this geometry
    assert call(T=1024) == 6
    assert call(out=FAKE + 16) == M.MOE_E_OVERLAP
    assert L.moe_workspace_bytes(32, 2048, 768, 128, 8, 1, M.F_PRENORM) <= 8 << 20
    assert L.moe_workspace_bytes(64, 2048, 768, 128, 8, 1, 0) > 8 << 20


def test_attn_prep_validation():
    L = M.lib()

    def W(**kw):
        base = dict(d_model=2048, n_q_heads=32, n_kv_heads=4, head_dim=128, format=0,
                    w_qkv=FAKE, attn_gain=FAKE, q_gain=FAKE, k_gain=FAKE)
        base.update(kw)
        return M.moe_attn_weights(**base)

    def call(w=None, T=1, x=FAKE, pos=FAKE, theta=1e6, q=FAKE, ws=FAKE, wsb=1 << 30, mp=8):
        w = W() if w is None else w
        return L.moe_attn_prep(x, T, ctypes.byref(w), pos, theta, 1e-6, q, FAKE, FAKE, mp, ws,
                               wsb, None)
    assert L.moe_attn_workspace_bytes(3, ctypes.byref(W())) == 256 + 3 * 5120 * 8 + 36 * 4
    assert call(T=0) == 0
    assert call(w=W(format=5)) == 4
    assert call(w=W(head_dim=100)) == 2
    assert call(w=W(d_model=100)) == 2
    assert call(w=W(d_model=4096)) == 6
    assert call(w=W(head_dim=512)) == 6
    assert call(theta=1.0) == 2
    assert call(x=None) == 1
    assert call(w=W(w_qkv=None)) == 1
    assert call(x=FAKE + 4) == 3
    assert call(wsb=100) == 5
    assert call() == M.MOE_E_OVERLAP        # x, q and both caches share one address here


def test_workspace_status_validation():
    L = M.lib()
    assert L.moe_workspace_status(None, 1 << 20, 0, None) == 1
    assert L.moe_workspace_status(FAKE, 67, 0, None) == 5


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "LIB_PATH", "/nonexistent/libmoe_mi355x.so")
    with pytest.raises(RuntimeError, match="missing"):
        M.lib()


def test_decode_stack_validation():
    L = M.lib()
    ex = _experts()

    def layers(*exs, gate=FAKE):
        return (M.moe_stack_layer * len(exs))(*[M.moe_stack_layer(gate, None, e) for e in exs])

    two = layers(ex, ex)

    def call(n=2, lay=two, k=8, flags=0, x=FAKE, outs=FAKE, ws=FAKE, wsb=1 << 40):
        return L.moe_decode_stack(x, n, lay, k, flags, outs, None, None, ws, wsb, None)

    assert call(n=0) == 2
    assert call(lay=None) == 1
    assert call(x=None) == 1
    assert call(outs=None) == 1
    assert call(flags=M.F_FP16_ACT) == 4
    assert call(k=0) == 2
    assert call(k=33) == 6
    assert call(x=FAKE + 2) == 3
    assert call(ws=None) == 5
    assert call(wsb=1000) == 5
    assert call(lay=layers(ex, _experts(d_ff=1536))) == 2
    assert call(lay=layers(ex, _experts(format=3))) == 4
    assert call(n=1, lay=layers(ex, gate=None)) == 1
    assert call(outs=FAKE - 2048 * 4) == M.MOE_E_OVERLAP                # x is o_1
