"""ctypes binding of libmoe_ep.so (the C ABI in include/moe_ep.h).

Argument marshalling only: torch tensors are checked for device, dtype,
contiguity and size against the shape, then their device pointers and the
current HIP stream are handed to the library.  Every step of the path runs in
the library's HIP kernels; there is no fallback.  Importing this module loads
the library and raises if it has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ep.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_CAPACITY = 2
MOE_ERR_UNSUPPORTED = 3
MOE_ERR_HIP = 4

MOE_BF16 = 0
MOE_FP8_E4M3 = 1
DTYPES = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}

MOE_GATE_SOFTMAX = 0
MOE_GATE_SIGMOID = 1
GATES = {"softmax": MOE_GATE_SOFTMAX, "sigmoid": MOE_GATE_SIGMOID}


class MoeShapeC(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("num_topk", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_ranks", ctypes.c_int32)]


class MoeRouterC(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_int32), ("num_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32)]


@dataclass(frozen=True)
class MoeShape:
    num_tokens: int
    hidden: int
    num_topk: int
    num_experts: int
    num_ranks: int

    def c(self) -> MoeShapeC:
        return MoeShapeC(self.num_tokens, self.hidden, self.num_topk, self.num_experts, self.num_ranks)


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python combine_get_dispatch_07_amd/build.py` "
                          "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    SH = ctypes.POINTER(MoeShapeC)
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_workspace_bytes.argtypes = [SH]
    lib.moe_workspace_bytes.restype = SZ
    lib.moe_max_recv_rows.argtypes = [SH]
    lib.moe_max_recv_rows.restype = I32
    lib.moe_get_dispatch_layout.argtypes = [SH, P, P, P, P, P, SZ, P]
    lib.moe_get_dispatch_layout.restype = ctypes.c_int
    lib.moe_route_layout.argtypes = [SH, ctypes.POINTER(MoeRouterC), P, P, P, P, P, P, P, SZ, P]
    lib.moe_route_layout.restype = ctypes.c_int
    lib.moe_route_dispatch.argtypes = [SH, ctypes.POINTER(MoeRouterC), ctypes.c_int, P, P, P, P, P, P, P, P, SZ, I32,
                                       P, P, P, P, P, P, P, P, P]
    lib.moe_route_dispatch.restype = ctypes.c_int
    lib.moe_dispatch.argtypes = [SH, ctypes.c_int, P, P, P, P, SZ, I32, P, P, P, P, P, P, P, P, P]
    lib.moe_dispatch.restype = ctypes.c_int
    lib.moe_combine.argtypes = [SH, P, I32, P, P, P, P, P]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_ll_workspace_bytes.argtypes = [SH]
    lib.moe_ll_workspace_bytes.restype = SZ
    lib.moe_dispatch_ll.argtypes = [SH, ctypes.c_int, P, P, P, SZ, I32, P, P, P, P, P, P]
    lib.moe_dispatch_ll.restype = ctypes.c_int
    lib.moe_combine_ll.argtypes = [SH, P, I32, P, P, P, P, P]
    lib.moe_combine_ll.restype = ctypes.c_int
    lib.moe_layout_dispatch.argtypes = [SH, ctypes.c_int, P, P, P, P, P, P, P, SZ, I32, P, P, P, P, P, P, P, P, P]
    lib.moe_layout_dispatch.restype = ctypes.c_int
    lib.moe_layout_dispatch_noalloc.argtypes = [SH, ctypes.c_int, P, P, P, P, P, P, I32, P, P, P, P, P, P, P, P, P]
    lib.moe_layout_dispatch_noalloc.restype = ctypes.c_int
    lib.moe_encode_e4m3.argtypes = [P, P, ctypes.c_int64, P]
    lib.moe_encode_e4m3.restype = ctypes.c_int
    lib.moe_combine_backward.argtypes = [SH, P, P, I32, P, P, P, P, P, P]
    lib.moe_combine_backward.restype = ctypes.c_int
    lib.moe_dispatch_backward.argtypes = [SH, P, I32, P, P, P, P, P, P]
    lib.moe_dispatch_backward.restype = ctypes.c_int
    lib.moe_stream_create_cu_range.argtypes = [I32, I32, ctypes.POINTER(ctypes.c_void_p)]
    lib.moe_stream_create_cu_range.restype = ctypes.c_int
    lib.moe_stream_destroy.argtypes = [P]
    lib.moe_stream_destroy.restype = ctypes.c_int
    return lib


lib = _load()


def status_string(code: int) -> str:
    return lib.moe_status_string(int(code)).decode()


def workspace_bytes(shape: MoeShape) -> int:
    return int(lib.moe_workspace_bytes(ctypes.byref(shape.c())))


def max_recv_rows(shape: MoeShape) -> int:
    return int(lib.moe_max_recv_rows(ctypes.byref(shape.c())))


def ll_workspace_bytes(shape: MoeShape) -> int:
    return int(lib.moe_ll_workspace_bytes(ctypes.byref(shape.c())))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype, numel: Optional[int] = None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _check(fn: str, code: int) -> None:
    if code != MOE_OK:
        raise MoeError(fn, code)


class Prepared:
    """One library call with its arguments checked and converted once: calling it launches the
    work on the given stream (default: torch's current stream).  It keeps the tensors it was
    prepared with alive; they must not be reallocated while it is in use.  For buffers allocated
    once and reused, as the exchange's are, this takes the per-call argument checks of the Python
    wrapper off the launch path (the library still checks every call on the host)."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name: str, fn, args, keep):
        self.name, self.fn, self.keep = name, fn, keep
        self.args = tuple(a if a is None or not isinstance(a, int) else t(a) for a, t in zip(args, fn.argtypes))

    def __call__(self, stream=None) -> None:
        code = self.fn(*self.args, _stream(stream))
        if code != MOE_OK:
            raise MoeError(self.name, code)


def _launch(name: str, args, stream, prepare: bool, scope: dict):
    """Calls library function `name` with `args` and the stream, or returns it as a Prepared call
    (keeping the tensors among the caller's arguments, `scope`, alive)."""
    fn = getattr(lib, name)
    if prepare:
        return Prepared(name, fn, args, tuple(v for v in scope.values() if isinstance(v, torch.Tensor)))
    _check(name, fn(*args, _stream(stream)))
    return None


def moe_get_dispatch_layout(shape: MoeShape, topk_idx, tokens_per_rank, tokens_per_expert, is_token_in_rank,
                            workspace, stream=None, prepare: bool = False):
    T, k, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
    return _launch("moe_get_dispatch_layout", (
        ctypes.byref(shape.c()), _ptr(topk_idx, "topk_idx", torch.int32, T * k),
        _ptr(tokens_per_rank, "tokens_per_rank", torch.int32, R),
        _ptr(tokens_per_expert, "tokens_per_expert", torch.int32, E),
        _ptr(is_token_in_rank, "is_token_in_rank", torch.uint8, T * R),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel()), stream, prepare, locals())


def moe_route_layout(shape: MoeShape, logits, topk_idx, topk_w, tokens_per_rank, tokens_per_expert,
                     is_token_in_rank, workspace, gate: str = "softmax", num_groups: int = 1, topk_groups: int = 1,
                     stream=None, prepare: bool = False):
    T, k, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
    router = MoeRouterC(GATES[gate], int(num_groups), int(topk_groups))
    return _launch("moe_route_layout", (
        ctypes.byref(shape.c()), ctypes.byref(router), _ptr(logits, "logits", torch.float32, T * E),
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(tokens_per_rank, "tokens_per_rank", torch.int32, R),
        _ptr(tokens_per_expert, "tokens_per_expert", torch.int32, E),
        _ptr(is_token_in_rank, "is_token_in_rank", torch.uint8, T * R),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel()), stream, prepare, locals())


def moe_route_dispatch(shape: MoeShape, dtype: str, logits, x, topk_idx, topk_w, tokens_per_rank, tokens_per_expert,
                       is_token_in_rank, workspace, recv_x, recv_scales, recv_src_idx, recv_topk_idx, recv_topk_w,
                       rank_offsets, send_row, num_recv, gate: str = "softmax", num_groups: int = 1,
                       topk_groups: int = 1, stream=None, prepare: bool = False):
    T, H, k, E, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts, shape.num_ranks
    fp8 = DTYPES[dtype] == MOE_FP8_E4M3
    cap = recv_src_idx.numel()
    router = MoeRouterC(GATES[gate], int(num_groups), int(topk_groups))
    return _launch("moe_route_dispatch", (
        ctypes.byref(shape.c()), ctypes.byref(router), DTYPES[dtype], _ptr(logits, "logits", torch.float32, T * E),
        _ptr(x, "x", torch.bfloat16, T * H),
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(tokens_per_rank, "tokens_per_rank", torch.int32, R),
        _ptr(tokens_per_expert, "tokens_per_expert", torch.int32, E),
        _ptr(is_token_in_rank, "is_token_in_rank", torch.uint8, T * R),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), cap,
        _ptr(recv_x, "recv_x", torch.uint8 if fp8 else torch.bfloat16, cap * H),
        _ptr(recv_scales, "recv_scales", torch.float32, cap * (H // 128)) if fp8 else None,
        _ptr(recv_src_idx, "recv_src_idx", torch.int32, cap),
        _ptr(recv_topk_idx, "recv_topk_idx", torch.int32, cap * k),
        _ptr(recv_topk_w, "recv_topk_w", torch.float32, cap * k),
        _ptr(rank_offsets, "rank_offsets", torch.int32, R + 1),
        _ptr(send_row, "send_row", torch.int32, T * R), _ptr(num_recv, "num_recv", torch.int32, 1)), stream, prepare, locals())


def moe_dispatch(shape: MoeShape, dtype: str, x, topk_idx, topk_w, workspace, recv_x, recv_scales, recv_src_idx,
                 recv_topk_idx, recv_topk_w, rank_offsets, send_row, num_recv, stream=None, prepare: bool = False):
    T, H, k, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_ranks
    fp8 = DTYPES[dtype] == MOE_FP8_E4M3
    cap = recv_src_idx.numel()
    return _launch("moe_dispatch", (
        ctypes.byref(shape.c()), DTYPES[dtype], _ptr(x, "x", torch.bfloat16, T * H),
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), cap,
        _ptr(recv_x, "recv_x", torch.uint8 if fp8 else torch.bfloat16, cap * H),
        _ptr(recv_scales, "recv_scales", torch.float32, cap * (H // 128)) if fp8 else None,
        _ptr(recv_src_idx, "recv_src_idx", torch.int32, cap),
        _ptr(recv_topk_idx, "recv_topk_idx", torch.int32, cap * k),
        _ptr(recv_topk_w, "recv_topk_w", torch.float32, cap * k),
        _ptr(rank_offsets, "rank_offsets", torch.int32, R + 1),
        _ptr(send_row, "send_row", torch.int32, T * R), _ptr(num_recv, "num_recv", torch.int32, 1)), stream, prepare, locals())


def moe_layout_dispatch(shape: MoeShape, dtype: str, x, topk_idx, topk_w, tokens_per_rank, tokens_per_expert,
                        is_token_in_rank, workspace, recv_x, recv_scales, recv_src_idx, recv_topk_idx, recv_topk_w,
                        rank_offsets, send_row, num_recv, stream=None, prepare: bool = False):
    T, H, k, E, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts, shape.num_ranks
    fp8 = DTYPES[dtype] == MOE_FP8_E4M3
    cap = recv_src_idx.numel()
    return _launch("moe_layout_dispatch", (
        ctypes.byref(shape.c()), DTYPES[dtype], _ptr(x, "x", torch.bfloat16, T * H),
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(tokens_per_rank, "tokens_per_rank", torch.int32, R),
        _ptr(tokens_per_expert, "tokens_per_expert", torch.int32, E),
        _ptr(is_token_in_rank, "is_token_in_rank", torch.uint8, T * R),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), cap,
        _ptr(recv_x, "recv_x", torch.uint8 if fp8 else torch.bfloat16, cap * H),
        _ptr(recv_scales, "recv_scales", torch.float32, cap * (H // 128)) if fp8 else None,
        _ptr(recv_src_idx, "recv_src_idx", torch.int32, cap),
        _ptr(recv_topk_idx, "recv_topk_idx", torch.int32, cap * k),
        _ptr(recv_topk_w, "recv_topk_w", torch.float32, cap * k),
        _ptr(rank_offsets, "rank_offsets", torch.int32, R + 1),
        _ptr(send_row, "send_row", torch.int32, T * R), _ptr(num_recv, "num_recv", torch.int32, 1)), stream, prepare, locals())


def moe_layout_dispatch_noalloc(shape: MoeShape, dtype: str, x, topk_idx, topk_w, tokens_per_rank,
                                tokens_per_expert, is_token_in_rank, recv_x, recv_scales, recv_src_idx, recv_topk_idx,
                                recv_topk_w, rank_offsets, send_row, num_recv, stream=None, prepare: bool = False):
    """moe_layout_dispatch with the plan in the library's static device array (no workspace)."""
    T, H, k, E, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts, shape.num_ranks
    fp8 = DTYPES[dtype] == MOE_FP8_E4M3
    cap = recv_src_idx.numel()
    return _launch("moe_layout_dispatch_noalloc", (
        ctypes.byref(shape.c()), DTYPES[dtype], _ptr(x, "x", torch.bfloat16, T * H),
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(tokens_per_rank, "tokens_per_rank", torch.int32, R),
        _ptr(tokens_per_expert, "tokens_per_expert", torch.int32, E),
        _ptr(is_token_in_rank, "is_token_in_rank", torch.uint8, T * R), cap,
        _ptr(recv_x, "recv_x", torch.uint8 if fp8 else torch.bfloat16, cap * H),
        _ptr(recv_scales, "recv_scales", torch.float32, cap * (H // 128)) if fp8 else None,
        _ptr(recv_src_idx, "recv_src_idx", torch.int32, cap),
        _ptr(recv_topk_idx, "recv_topk_idx", torch.int32, cap * k),
        _ptr(recv_topk_w, "recv_topk_w", torch.float32, cap * k),
        _ptr(rank_offsets, "rank_offsets", torch.int32, R + 1),
        _ptr(send_row, "send_row", torch.int32, T * R), _ptr(num_recv, "num_recv", torch.int32, 1)), stream, prepare, locals())


def moe_combine(shape: MoeShape, y, topk_idx, topk_w, send_row, out, stream=None, prepare: bool = False, num_y_rows=None):
    T, H, k, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_ranks
    rows = y.shape[0] if num_y_rows is None else int(num_y_rows)
    return _launch("moe_combine", (
        ctypes.byref(shape.c()), _ptr(y, "y", torch.bfloat16, rows * H), rows,
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(send_row, "send_row", torch.int32, T * R), _ptr(out, "out", torch.bfloat16, T * H)), stream, prepare, locals())


def moe_dispatch_ll(shape: MoeShape, dtype: str, x, topk_idx, workspace, recv_x, recv_scales, recv_src_idx,
                    recv_count, slot_pos, stream=None, prepare: bool = False):
    T, H, k, E = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts
    fp8 = DTYPES[dtype] == MOE_FP8_E4M3
    cap = recv_src_idx.shape[1] if recv_src_idx.dim() == 2 else recv_src_idx.numel() // max(E, 1)
    return _launch("moe_dispatch_ll", (
        ctypes.byref(shape.c()), DTYPES[dtype], _ptr(x, "x", torch.bfloat16, T * H),
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(workspace, "workspace", torch.uint8),
        workspace.numel(), cap, _ptr(recv_x, "recv_x", torch.uint8 if fp8 else torch.bfloat16, E * cap * H),
        _ptr(recv_scales, "recv_scales", torch.float32, E * cap * (H // 128)) if fp8 else None,
        _ptr(recv_src_idx, "recv_src_idx", torch.int32, E * cap), _ptr(recv_count, "recv_count", torch.int32, E),
        _ptr(slot_pos, "slot_pos", torch.int32, T * k)), stream, prepare, locals())


def moe_combine_ll(shape: MoeShape, y, topk_idx, topk_w, slot_pos, out, stream=None, prepare: bool = False):
    T, H, k, E = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts
    cap = y.shape[1]
    return _launch("moe_combine_ll", (
        ctypes.byref(shape.c()), _ptr(y, "y", torch.bfloat16, E * cap * H), cap,
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(slot_pos, "slot_pos", torch.int32, T * k), _ptr(out, "out", torch.bfloat16, T * H)), stream, prepare, locals())


def moe_encode_e4m3(values, codes, stream=None, prepare: bool = False):
    """codes (uint8) = E4M3 round-to-nearest-even codes of values (float32), as the FP8 dispatch
    rounds x / s; defined for finite |values| < 464."""
    n = values.numel()
    if codes.numel() != n:
        raise ValueError(f"codes: {codes.numel()} elements for {n} values")
    return _launch("moe_encode_e4m3", (_ptr(values, "values", torch.float32, n), _ptr(codes, "codes", torch.uint8, n),
                                       n), stream, prepare, locals())


def moe_combine_backward(shape: MoeShape, grad_out, y, topk_idx, topk_w, send_row, grad_y, grad_topk_w,
                         stream=None, prepare: bool = False, num_y_rows=None):
    T, H, k, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_ranks
    rows = y.shape[0] if num_y_rows is None else int(num_y_rows)
    return _launch("moe_combine_backward", (
        ctypes.byref(shape.c()), _ptr(grad_out, "grad_out", torch.bfloat16, T * H),
        _ptr(y, "y", torch.bfloat16, rows * H), rows, _ptr(topk_idx, "topk_idx", torch.int32, T * k),
        _ptr(topk_w, "topk_w", torch.float32, T * k), _ptr(send_row, "send_row", torch.int32, T * R),
        _ptr(grad_y, "grad_y", torch.bfloat16, rows * H), _ptr(grad_topk_w, "grad_topk_w", torch.float32, T * k)), stream, prepare, locals())


def moe_dispatch_backward(shape: MoeShape, grad_recv_x, topk_idx, send_row, grad_x, grad_recv_topk_w=None,
                          grad_topk_w=None, stream=None, prepare: bool = False, num_recv_rows=None):
    T, H, k, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_ranks
    rows = grad_recv_x.shape[0] if num_recv_rows is None else int(num_recv_rows)
    return _launch("moe_dispatch_backward", (
        ctypes.byref(shape.c()), _ptr(grad_recv_x, "grad_recv_x", torch.bfloat16, rows * H), rows,
        _ptr(grad_recv_topk_w, "grad_recv_topk_w", torch.float32, rows * k),
        _ptr(topk_idx, "topk_idx", torch.int32, T * k), _ptr(send_row, "send_row", torch.int32, T * R),
        _ptr(grad_x, "grad_x", torch.bfloat16, T * H), _ptr(grad_topk_w, "grad_topk_w", torch.float32, T * k)), stream, prepare, locals())


def stream_create_cu_range(first_cu: int, num_cus: int) -> int:
    """A HIP stream restricted to CUs [first_cu, first_cu + num_cus); returns its handle."""
    h = ctypes.c_void_p()
    _check("moe_stream_create_cu_range", lib.moe_stream_create_cu_range(int(first_cu), int(num_cus), ctypes.byref(h)))
    return int(h.value or 0)


def stream_destroy(handle: int) -> None:
    _check("moe_stream_destroy", lib.moe_stream_destroy(ctypes.c_void_p(handle)))
