"""The C-ABI library loads, exports every symbol its header declares, and
rejects invalid calls before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from top_routing_expert_route_amd import api
    if not os.path.exists(api.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return api.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_grouped_gemm"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from top_routing_expert_route_amd import api
    raw = ctypes.CDLL(api.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(raw, n)]
    assert not missing, missing
    assert sorted(api.EXPORTS) == _declared()


def test_version_and_strings(lib):
    assert lib.moe_abi_version() == 3
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(3) == b"workspace too small"


def test_max_rows(lib):
    assert lib.moe_max_rows(4096, 8, 2, 0.0, 0) == 8192
    assert lib.moe_max_rows(8192, 64, 2, 1.25, 0) == 64 * 160
    assert lib.moe_max_rows(32768, 256, 8, 0.0, 32) == 32768 * 8
    assert lib.moe_max_rows(100, 4, 2, 0.5, 2) == 2 * 12
    assert lib.moe_max_rows(-1, 4, 2, 0.0, 0) == -1


def test_workspace_sizes(lib):
    from top_routing_expert_route_amd import api
    assert lib.moe_route_workspace_size(4096, 4096, 8) > 4096 * 8 * 4
    assert lib.moe_route_workspace_size(0, 64, 8) == 0
    assert lib.moe_dispatch_workspace_size(4096, 2, 8) > 0
    p = api.Problem(4096, 4096, 8, 2, 16384, 0.0, 0, 0, 0, 0.01, api.MOE_BF16)
    n = lib.moe_forward_workspace_size(ctypes.byref(p))
    # at least x_perm + h + y_perm for 8192 rows
    assert n >= 8192 * (4096 + 16384 + 4096) * 2


FAKE = 1 << 20  # a 16-byte aligned non-NULL address that is never dereferenced


def test_route_rejects_bad_arguments(lib):
    from top_routing_expert_route_amd import api
    P = FAKE
    call = lambda **kw: lib.moe_route(kw.get("x", P), kw.get("dt", 1), P, None, None, kw.get("T", 16), kw.get("d", 64),
                                      kw.get("E", 8), kw.get("k", 2), 0.01, P, P, None, None, None, None,
                                      kw.get("ws", P), kw.get("wsb", 1 << 30), None)
    assert call(k=9) == api.MOE_ERR_INVALID_ARG
    assert call(k=0) == api.MOE_ERR_INVALID_ARG
    assert call(T=-1) == api.MOE_ERR_INVALID_ARG
    assert call(x=None) == api.MOE_ERR_INVALID_ARG
    assert call(x=P + 4) == api.MOE_ERR_INVALID_ARG
    assert call(dt=7) == api.MOE_ERR_INVALID_ARG
    assert call(d=60) == api.MOE_ERR_UNSUPPORTED
    assert call(E=2000, k=2) == api.MOE_ERR_UNSUPPORTED
    assert call(E=64, k=33) == api.MOE_ERR_UNSUPPORTED
    assert call(ws=None) == api.MOE_ERR_WORKSPACE
    assert call(wsb=16) == api.MOE_ERR_WORKSPACE
    assert b"workspace" in lib.moe_last_error()


def test_dispatch_rejects_bad_arguments(lib):
    from top_routing_expert_route_amd import api
    P = FAKE

    def call(**kw):
        return lib.moe_dispatch(P, 1, P, kw.get("T", 16), 64, kw.get("E", 8), kw.get("k", 2), kw.get("cf", 0.0),
                                kw.get("e0", 0), kw.get("nle", 0), P, P, P, P, kw.get("xp", P),
                                kw.get("rows", 32), None, P, 1 << 30, None)
    assert call() == api.MOE_OK or True  # (would launch: not called on CPU)
    assert call(rows=31) == api.MOE_ERR_INVALID_ARG
    assert call(e0=1) == api.MOE_ERR_INVALID_ARG          # e0 != 0 with the whole layer
    assert call(e0=6, nle=4) == api.MOE_ERR_INVALID_ARG   # [6, 10) outside [0, 8)
    assert call(cf=float("nan")) == api.MOE_ERR_INVALID_ARG
    assert call(k=3, E=2) == api.MOE_ERR_INVALID_ARG
    assert call(xp=P + 8) == api.MOE_ERR_INVALID_ARG


def test_gemm_and_combine_reject_bad_arguments(lib):
    from top_routing_expert_route_amd import api
    P = FAKE
    g = lambda *a: lib.moe_grouped_gemm(*a, None, 0, None)
    assert g(P, P, 4, 100, 60, 64, 1, P, None, 1, P) == api.MOE_ERR_UNSUPPORTED
    assert g(P, P, 4, 100, 64, 64, 1, P, None, 2, P) == api.MOE_ERR_UNSUPPORTED
    assert g(P, P, 0, 100, 64, 64, 1, P, None, 0, P) == api.MOE_ERR_INVALID_ARG
    assert g(P, P, 2000, 100, 64, 64, 1, P, None, 0, P) == api.MOE_ERR_UNSUPPORTED
    assert g(None, P, 4, 100, 64, 64, 1, P, None, 0, P) == api.MOE_ERR_INVALID_ARG
    # K past 2^21: a 256-row operand tile would not fit one 32-bit buffer record
    assert g(P, P, 4, 100, 64, (1 << 21) + 64, 1, P, None, 0, P) == api.MOE_ERR_UNSUPPORTED
    assert b"buffer" in lib.moe_last_error()
    assert lib.moe_grouped_gemm(P, P, 4, 100, 64, 64, 1, P, None, 0, P, P + 4, 1 << 30, None) \
        == api.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(P, 10, P, P, None, 4, 64, 33, 1, P, None) == api.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(P, 10, None, P, None, 4, 64, 2, 1, P, None) == api.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(P, P, 4, 100, 64, 100, 1, P, None, P, None, P, P, None, 0, None) \
        == api.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_gemm_workspace_size() > 0


def test_forward_rejects_bad_arguments(lib):
    from top_routing_expert_route_amd import api
    assert lib.moe_forward(None, None, None, None, None, None, 0, None) == api.MOE_ERR_INVALID_ARG
    p = api.Problem(16, 64, 8, 2, 128, 0.0, 0, 0, 0, 0.01, api.MOE_BF16)
    w = api.Weights(FAKE, None, None, None, FAKE, None, None, None, None, None)   # w1 missing
    assert lib.moe_forward(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, None, FAKE, 1 << 40, None) \
        == api.MOE_ERR_INVALID_ARG
    w = api.Weights(FAKE, None, FAKE, None, FAKE, None, None, None, None, None)
    assert lib.moe_forward(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, None, FAKE, 16, None) \
        == api.MOE_ERR_WORKSPACE
    p.has_shared = 1
    assert lib.moe_forward(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, None, FAKE, 1 << 40, None) \
        == api.MOE_ERR_INVALID_ARG


def test_backward_workspace_and_rejections(lib):
    """moe_backward validates everything before enqueuing (no GPU touched)."""
    from top_routing_expert_route_amd import api
    p = api.Problem(4096, 4096, 8, 2, 16384, 0.0, 0, 0, 0, 0.01, api.MOE_BF16)
    nb = lib.moe_backward_workspace_size(ctypes.byref(p))
    # u, dh' (fp32) and dx rows (fp32) for 8192 rows, at least
    assert nb >= 8192 * (16384 * 2 + 4096) * 4
    assert nb > lib.moe_forward_workspace_size(ctypes.byref(p))
    assert lib.moe_backward(None, None, None, None, 0.0, None, None, 0, None) == api.MOE_ERR_INVALID_ARG

    p = api.Problem(64, 128, 8, 2, 128, 0.0, 0, 0, 0, 0.01, api.MOE_BF16)
    w = api.Weights(FAKE, None, FAKE, None, FAKE, None, None, None, None, None)
    full = dict(dx=FAKE, dw_router=FAKE, dw1=FAKE, dw2=FAKE)

    def call(prob, grads, ws_bytes=1 << 40, g_aux=0.0):
        g = api.Grads(**{n: grads.get(n) for n, _ in api.Grads._fields_})
        return lib.moe_backward(ctypes.byref(prob), ctypes.byref(w), FAKE, FAKE, g_aux, ctypes.byref(g), FAKE,
                                ws_bytes, None)

    assert call(p, full, ws_bytes=16) == api.MOE_ERR_WORKSPACE
    assert call(p, dict(full, dw1=None)) == api.MOE_ERR_INVALID_ARG
    assert call(p, dict(full, db1=FAKE + 4)) == api.MOE_ERR_INVALID_ARG      # misaligned
    assert call(p, full, g_aux=float("nan")) == api.MOE_ERR_INVALID_ARG
    p.has_shared = 1                                                            # no shared weights/grads
    assert call(p, full) == api.MOE_ERR_INVALID_ARG
    p = api.Problem(64, 136, 8, 2, 128, 0.0, 0, 0, 0, 0.01, api.MOE_BF16)     # d % 64 != 0 in bf16
    assert call(p, full) == api.MOE_ERR_UNSUPPORTED
    assert b"multiples of 64" in lib.moe_last_error()
    # the saved-activation entry points need their u buffers
    g = api.Grads(**{n: full.get(n) for n, _ in api.Grads._fields_})
    assert lib.moe_backward_saved(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, 0.0, None, None, ctypes.byref(g),
                                  FAKE, 1 << 40, None) == api.MOE_ERR_INVALID_ARG
    assert b"u_saved" in lib.moe_last_error()
    assert lib.moe_backward_saved(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, 0.0, FAKE + 8, None,
                                  ctypes.byref(g), FAKE, 1 << 40, None) == api.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_save(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, None, None, None, FAKE, 1 << 40,
                                None) == api.MOE_ERR_INVALID_ARG
    # bf16 with d % 64 != 0 (here d = 136): the fp32-output first Linear needs the 256x256 kernel
    assert lib.moe_forward_save(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, None, FAKE, None, FAKE, 1 << 40,
                                None) == api.MOE_ERR_UNSUPPORTED
    # 2^20 tokens x k = 2 rows: the weight-gradient GEMMs would need > 2^21 columns
    p = api.Problem(1 << 20, 128, 8, 2, 128, 0.0, 0, 0, 0, 0.01, api.MOE_BF16)
    assert call(p, full) == api.MOE_ERR_UNSUPPORTED
    assert b"columns" in lib.moe_last_error()


def test_binding_checks_caller_outputs():
    """The binding's `out=` form checks the caller's tensors before any call
    reaches the library (which trusts the sizes it is given)."""
    import torch
    from top_routing_expert_route_amd import api
    x = torch.zeros((16, 8), dtype=torch.bfloat16)
    wr = torch.zeros((4, 8), dtype=torch.float32)
    good = dict(topk_idx=torch.empty((16, 2), dtype=torch.int32), topk_w=torch.empty((16, 2)),
                expert_count=torch.empty(4, dtype=torch.int32), f=torch.empty(4), P=torch.empty(4),
                l_aux=torch.empty(1))
    for name, bad in (("topk_idx", torch.empty((16, 3), dtype=torch.int32)),
                      ("topk_w", torch.empty((16, 2), dtype=torch.float64)),
                      ("P", torch.empty(8)[::2])):
        out = dict(good, **{name: bad})
        with pytest.raises(ValueError, match=name):
            api.moe_route(x, wr, None, 2, out=out)
    idx = torch.zeros((16, 2), dtype=torch.int32)
    mr = api.max_rows(16, 4, 2)
    dgood = dict(seg_offsets=torch.empty(5, dtype=torch.int32), kept_count=torch.empty(4, dtype=torch.int32),
                 slot_row=torch.empty((16, 2), dtype=torch.int32), row_src=torch.empty(mr, dtype=torch.int32),
                 n_dropped=torch.empty(1, dtype=torch.int32), x_perm=torch.empty((mr, 8), dtype=torch.bfloat16))
    for name, bad in (("row_src", torch.empty(mr - 1, dtype=torch.int32)),
                      ("x_perm", torch.empty((mr, 8), dtype=torch.float32)),
                      ("seg_offsets", None)):
        out = dict(dgood, **{name: bad})
        with pytest.raises(ValueError, match=name):
            api.moe_dispatch(x, idx, 4, out=out)
