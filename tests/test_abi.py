"""The C-ABI library: it loads, exports every symbol include/moe_ep.h declares,
and rejects bad arguments on the host with the documented status codes before
anything is launched (no GPU needed: every call here fails validation, or has
nothing to launch)."""
import ctypes
import os
import re

import pytest

from combine_get_dispatch_07_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_ep.h")

OK, INVALID, CAPACITY, UNSUPPORTED = L.MOE_OK, L.MOE_ERR_INVALID_ARG, L.MOE_ERR_CAPACITY, L.MOE_ERR_UNSUPPORTED
A = 0x100000  # a fake, well aligned device address: validation never dereferences it


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"moe_get_dispatch_layout", "moe_dispatch", "moe_combine", "moe_workspace_bytes",
                          "moe_max_recv_rows", "moe_status_string"}
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def shape(T=64, H=256, k=4, E=16, R=4):
    return L.MoeShapeC(T, H, k, E, R)


def layout(s, topk=A, tpr=A, tpe=A, mask=A, ws=A, ws_bytes=1 << 30):
    return L.lib.moe_get_dispatch_layout(ctypes.byref(s) if s is not None else None, topk, tpr, tpe, mask, ws,
                                         ws_bytes, None)


def dispatch(s, dtype=0, cap=None, x=A, scales=A, ws=A, ws_bytes=1 << 30, recv_x=A, **kw):
    if cap is None:
        cap = s.num_tokens * min(s.num_topk, s.num_ranks)
    p = dict(topk=A, w=A, src=A, ridx=A, rw=A, offs=A, send=A, n=A)
    p.update(kw)
    return L.lib.moe_dispatch(ctypes.byref(s), dtype, x, p["topk"], p["w"], ws, ws_bytes, cap, recv_x, scales,
                              p["src"], p["ridx"], p["rw"], p["offs"], p["send"], p["n"], None)


def combine(s, y=A, rows=10, out=A, topk=A, w=A, send=A):
    return L.lib.moe_combine(ctypes.byref(s), y, rows, topk, w, send, out, None)


def test_status_strings():
    for code, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARG"), (2, "MOE_ERR_CAPACITY"),
                       (3, "MOE_ERR_UNSUPPORTED"), (4, "MOE_ERR_HIP")]:
        assert L.status_string(code) == name
    assert L.status_string(99) == "MOE_ERR_UNKNOWN"


def test_sizes():
    assert L.max_recv_rows(L.MoeShape(4096, 7168, 8, 256, 8)) == 4096 * 8
    assert L.max_recv_rows(L.MoeShape(100, 256, 8, 16, 4)) == 400
    assert L.max_recv_rows(L.MoeShape(100, 256, 8, 16, 3)) == -1  # E % R != 0
    ws = L.workspace_bytes(L.MoeShape(4096, 7168, 8, 256, 8))
    # sync words + expert and rank accumulators + token bitmasks + chunk rows + offsets, each 256-aligned
    assert ws >= 4 * 4096 + 256 * 4 + 8 * 4 + 4096 * 8 + 8 * 64 * 4 + 9 * 4 and ws % 256 == 0
    assert L.workspace_bytes(L.MoeShape(0, 256, 1, 4, 4)) > 0
    assert L.workspace_bytes(L.MoeShape(-1, 256, 1, 4, 4)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(H=0), INVALID), (dict(H=12), INVALID), (dict(k=0), INVALID),
    (dict(E=0), INVALID), (dict(R=0), INVALID), (dict(E=16, R=3), INVALID), (dict(E=4, R=8), INVALID),
    (dict(k=5, E=4, R=4), INVALID), (dict(k=33, E=64), UNSUPPORTED), (dict(R=128, E=256), UNSUPPORTED),
    (dict(E=8192, R=8), UNSUPPORTED), (dict(T=(1 << 30) + 1, k=1, E=1, R=1), UNSUPPORTED),
])
def test_shape_errors(kw, code):
    s = shape(**kw)
    assert layout(s) == code
    assert dispatch(s) == code
    assert combine(s) == code


def test_layout_errors():
    s = shape()
    need = L.lib.moe_workspace_bytes(ctypes.byref(s))
    assert layout(None) == INVALID
    for name in ("topk", "tpr", "tpe", "mask", "ws"):
        assert layout(s, **{name: None}) == INVALID, name
    assert layout(s, topk=A + 2) == INVALID
    assert layout(s, ws=A + 16) == INVALID  # the plan needs 256-byte alignment
    assert layout(s, ws_bytes=need - 1) == INVALID


def test_dispatch_errors():
    s = shape()
    cap = 64 * 4
    assert dispatch(s, dtype=2) == INVALID
    assert dispatch(s, cap=cap - 1) == CAPACITY
    assert dispatch(s, cap=-1) == INVALID
    assert dispatch(s, x=A + 8) == INVALID  # payload needs 16-byte alignment
    assert dispatch(s, recv_x=A + 4) == INVALID
    assert dispatch(s, ws_bytes=16) == INVALID
    for name in ("topk", "w", "src", "ridx", "rw", "offs", "send", "n"):
        assert dispatch(s, **{name: None}) == INVALID, name
    assert dispatch(s, dtype=1, scales=None) == INVALID  # fp8 needs the scale array
    assert dispatch(shape(H=136), dtype=1) == INVALID    # fp8 needs H % 128 == 0
    # R > k: capacity is T * k
    s2 = shape(T=10, k=2, E=16, R=8)
    assert dispatch(s2, cap=19) == CAPACITY


def test_combine_errors_and_empty():
    s = shape()
    assert combine(s, rows=-1) == INVALID
    assert combine(s, y=None) == INVALID
    assert combine(s, y=A + 2) == INVALID
    assert combine(s, out=A + 4) == INVALID
    assert combine(shape(T=0)) == OK  # nothing to launch
    # empty arrays may be NULL (torch gives zero-size tensors a null pointer)
    assert combine(shape(T=0), y=None, rows=0, out=None, topk=None, w=None, send=None) == OK
    assert combine(shape(T=5), out=None) == INVALID  # five tokens need an output array


def test_binding_rejects_host_tensors():
    import torch
    s = L.MoeShape(4, 256, 2, 8, 2)
    with pytest.raises(ValueError):
        L.moe_combine(s, torch.zeros(8, 256, dtype=torch.bfloat16), torch.zeros(4, 2, dtype=torch.int32),
                      torch.zeros(4, 2), torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 256, dtype=torch.bfloat16),
                      stream=0)


def route(s, gate=0, G=1, KG=1, router=True, logits=A, idx=A, w=A, tpr=A, tpe=A, mask=A, ws=A, ws_bytes=1 << 30):
    r = L.MoeRouterC(gate, G, KG)
    return L.lib.moe_route_layout(ctypes.byref(s), ctypes.byref(r) if router else None, logits, idx, w, tpr, tpe,
                                  mask, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,shape_kw,code", [
    (dict(router=False), {}, INVALID),
    (dict(gate=2), {}, INVALID),
    (dict(gate=-1), {}, INVALID),
    (dict(G=0), {}, INVALID),
    (dict(G=4, KG=5), {}, INVALID),
    (dict(G=4, KG=0), {}, INVALID),
    (dict(G=3, KG=1), dict(E=24, R=4), UNSUPPORTED),      # groups must be 1, 2, 4 or 8
    (dict(G=16, KG=2), dict(E=64, R=4), UNSUPPORTED),
    (dict(G=8, KG=1), dict(E=16, k=4, R=4), INVALID),      # k > topk_groups * E / G = 2
    (dict(), dict(E=12, R=4, k=4), UNSUPPORTED),           # E % 8 != 0
    (dict(), dict(E=4104, R=8, k=8), UNSUPPORTED),         # E above the library limit
    (dict(), dict(E=64, R=8, k=17), UNSUPPORTED),          # k > 16
    (dict(logits=0), {}, INVALID),
    (dict(idx=0), {}, INVALID),
    (dict(w=0), {}, INVALID),
    (dict(tpr=0), {}, INVALID),
    (dict(ws=A + 64), {}, INVALID),                        # workspace not 256-byte aligned
    (dict(ws_bytes=16), {}, INVALID),
    (dict(logits=A + 2), {}, INVALID),
])
def test_route_layout_rejects(kw, shape_kw, code):
    assert route(shape(**shape_kw), **kw) == code


def test_encode_e4m3_rejections():
    enc = L.lib.moe_encode_e4m3
    assert enc(A, A, -1, None) == INVALID
    assert enc(None, A, 4, None) == INVALID
    assert enc(A, None, 4, None) == INVALID
    assert enc(None, None, 0, None) == OK  # nothing to launch


def test_layout_dispatch_rejections():
    """The union of the layout's and the dispatch's checks, before any launch."""
    fn = L.lib.moe_layout_dispatch
    s = shape()
    cap = s.num_tokens * min(s.num_topk, s.num_ranks)

    def call(dtype=0, ws=A, ws_bytes=1 << 30, cap_=cap, mask=A, x=A, scales=A):
        return fn(ctypes.byref(s), dtype, x, A, A, A, A, mask, ws, ws_bytes, cap_, A, scales, A, A, A, A, A, A, None)

    assert call(dtype=7) == INVALID
    assert call(cap_=cap - 1) == CAPACITY
    assert call(ws_bytes=1) == INVALID
    assert call(mask=None) == INVALID  # a layout output missing
    assert call(x=A + 2) == INVALID  # misaligned x
    assert call(dtype=1, scales=None) == INVALID  # FP8 needs scales
    assert fn(None, 0, A, A, A, A, A, A, A, 1 << 30, cap, A, A, A, A, A, A, A, A, None) == INVALID


def test_layout_dispatch_noalloc_rejections():
    """The no-allocation variant checks what moe_layout_dispatch checks, and rejects shapes whose
    plan does not fit its 4 MiB static array, before any launch."""
    fn = L.lib.moe_layout_dispatch_noalloc
    s = shape()
    cap = s.num_tokens * min(s.num_topk, s.num_ranks)

    def call(sh=s, dtype=0, cap_=cap, mask=A, x=A, scales=A):
        return fn(ctypes.byref(sh), dtype, x, A, A, A, A, mask, cap_, A, scales, A, A, A, A, A, A, None)

    assert call(dtype=7) == INVALID
    assert call(cap_=cap - 1) == CAPACITY
    assert call(mask=None) == INVALID
    assert call(x=A + 2) == INVALID
    assert call(dtype=1, scales=None) == INVALID
    big = L.MoeShape(1 << 20, 256, 8, 256, 64).c()  # plan: 8 MiB of token bitmasks alone
    assert L.lib.moe_workspace_bytes(ctypes.byref(big)) > 4 << 20
    assert call(sh=big, cap_=(1 << 20) * 8) == UNSUPPORTED
    ok = L.MoeShape(300000, 256, 8, 256, 64).c()  # the documented reach: about 300,000 tokens
    assert L.lib.moe_workspace_bytes(ctypes.byref(ok)) <= 4 << 20
    assert fn(None, 0, A, A, A, A, A, A, cap, A, A, A, A, A, A, A, A, None) == INVALID


def test_prepared_call_checks_its_tensors_once_at_prepare_time():
    """prepare=True runs the wrapper's tensor checks up front (CPU tensors are refused) and
    converts the remaining integer arguments to the declared ctypes types."""
    import torch
    sh = L.MoeShape(8, 256, 4, 16, 4)
    with pytest.raises(ValueError):
        L.moe_combine(sh, torch.zeros(8, 256, dtype=torch.bfloat16), torch.zeros(8, 4, dtype=torch.int32),
                      torch.zeros(8, 4), torch.zeros(8, 4, dtype=torch.int32),
                      torch.zeros(8, 256, dtype=torch.bfloat16), prepare=True)
    p = L.Prepared("moe_encode_e4m3", L.lib.moe_encode_e4m3, (A, A, 0), ())
    assert isinstance(p.args[2], ctypes.c_int64) and p.args[0].value == A
