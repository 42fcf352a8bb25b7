"""ctypes binding of libmoe_route.so (include/moe_route.h), with the C names.

Argument marshalling only: torch tensors supply device memory and the current HIP stream, and
every step runs in the library's HIP kernels. If the library is not built, loading fails with an
ImportError; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_route.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_MAX_EXPERTS = 1024
MOE_MAX_TOPK = 64
MOE_NOALLOC_SCRATCH_BYTES = 16 << 20

DTYPE_CODES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8_e4m3": MOE_FP8_E4M3}
TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {moe_status_str(status)}")
        self.status = status


class moe_dispatch_out_t(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "recv", "recv_scales", "expert_counts", "expert_offsets", "rank_counts", "rank_offsets",
        "token_row", "row_token")]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.moe_status_str.argtypes = [I]
        lib.moe_status_str.restype = ctypes.c_char_p
        lib.moe_route_topk.argtypes = [P, I, I, I, P, P, P]
        lib.moe_dispatch_workspace_bytes.argtypes = [I, I, I]
        lib.moe_dispatch_workspace_bytes.restype = Z
        lib.moe_dispatch_layout.argtypes = [P, I, I, I, I, P, P, Z, P]
        lib.moe_dispatch_pack.argtypes = [P, I, I, I, I, P, I, P, P, P]
        lib.moe_dispatch.argtypes = [P, I, I, I, P, I, I, I, I, P, P, Z, P]
        lib.moe_route_dispatch.argtypes = [P, P, I, I, I, I, I, I, I, P, P, P, P, Z, P]
        lib.moe_route_dispatch_noalloc.argtypes = [P, P, I, I, I, I, I, I, I, P, P, P, P]
        lib.moe_combine.argtypes = [P, I, I, I, I, P, P, P, I, P]
        lib.moe_ep_capacity.argtypes = [I, I, I, I]
        lib.moe_ep_capacity.restype = ctypes.c_int64
        lib.moe_ep_send.argtypes = [P, I, I, I, P, I, I, I, I, I, I, P, P, P, P, Z, P]
        lib.moe_ep_recv.argtypes = [P, I, I, I, I, I, I, I, P, P, P, P, P, P]
        lib.moe_ep_return.argtypes = [P, I, I, I, I, I, I, P, P, P, P]
        lib.moe_ep_combine.argtypes = [P, I, I, I, I, P, P, I, P, I, P]
        lib.moe_ep_partial_rows.argtypes = [P, I, I, I, I, I, I, I, P, P, P]
        lib.moe_ep_reduce_workspace_bytes.argtypes = [I, I]
        lib.moe_ep_reduce_workspace_bytes.restype = Z
        lib.moe_ep_reduce.argtypes = [P, I, I, I, I, I, I, I, P, I, I, P, P, P, P, I, P, P, Z, P]
        lib.moe_ep_combine_reduced.argtypes = [P, I, I, I, I, P, I, P, I, P]
        lib.moe_check_topk.argtypes = [P, I, I, I, P, P]
        for fn in ("moe_route_topk", "moe_dispatch_layout", "moe_dispatch_pack", "moe_dispatch",
                   "moe_route_dispatch", "moe_route_dispatch_noalloc", "moe_combine", "moe_ep_send", "moe_ep_recv",
                   "moe_ep_return", "moe_ep_combine", "moe_ep_partial_rows", "moe_ep_reduce",
                   "moe_ep_combine_reduced", "moe_check_topk"):
            getattr(lib, fn).restype = I
        _lib = lib
    return _lib


def moe_status_str(status: int) -> str:
    return load().moe_status_str(status).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor, fp8_ok: bool = False) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if fp8_ok and t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def moe_route_topk(logits: torch.Tensor, k: int, topk_idx: Optional[torch.Tensor] = None,
                   topk_w: Optional[torch.Tensor] = None, stream=None):
    """Top-k expert ids (int32 [T,k]) and renormalised softmax weights (fp32 [T,k])."""
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    assert logits.dtype == torch.float32 and logits.is_contiguous()
    _check("moe_route_topk", load().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx),
                                                   _ptr(topk_w), _stream(stream)))
    return topk_idx, topk_w


def moe_check_topk(topk_idx: torch.Tensor, E: int, counts: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Device int32 [2]: slots with an id outside [0, E), in-range slots repeating an earlier slot
    of their token. Enqueued on the stream; read it after the stream has finished."""
    T, k = topk_idx.shape
    if counts is None:
        counts = torch.empty(2, dtype=torch.int32, device=topk_idx.device)
    assert topk_idx.dtype == torch.int32 and topk_idx.is_contiguous()
    _check("moe_check_topk", load().moe_check_topk(_ptr(topk_idx), T, k, E, _ptr(counts),
                                                   _stream(stream)))
    return counts


def _debug_check_ids(fn: str, topk_idx: torch.Tensor, E: int, stream) -> None:
    """With MOE_ROUTE_DEBUG=1, check caller-given ids on the GPU before they are dispatched and
    raise ValueError naming what is wrong (this waits for the stream)."""
    if os.environ.get("MOE_ROUTE_DEBUG", "0") != "1":
        return
    counts = moe_check_topk(topk_idx, E, stream=stream)
    bad, rep = (int(v) for v in counts.cpu().tolist())
    if bad or rep:
        raise ValueError(f"{fn}: {bad} expert ids outside [0, {E}) and {rep} repeated within a "
                         f"token (MOE_ROUTE_DEBUG=1)")


def moe_dispatch_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(load().moe_dispatch_workspace_bytes(T, E, k))


@dataclass
class DispatchBuffers:
    """Caller-owned dispatch outputs (device tensors)."""
    recv: Optional[torch.Tensor]
    recv_scales: Optional[torch.Tensor]
    expert_counts: torch.Tensor
    expert_offsets: torch.Tensor
    rank_counts: torch.Tensor
    rank_offsets: torch.Tensor
    token_row: torch.Tensor
    row_token: torch.Tensor

    def as_struct(self) -> moe_dispatch_out_t:
        s = moe_dispatch_out_t()
        for name, _ in moe_dispatch_out_t._fields_:
            t = getattr(self, name)
            setattr(s, name, None if t is None else t.data_ptr())
        return s


def alloc_dispatch_out(T: int, H: int, E: int, k: int, N: int, payload: Optional[str],
                       device="cuda") -> DispatchBuffers:
    """Allocate the outputs of one dispatch (payload None: layout outputs only)."""
    R = T * k
    i32 = dict(dtype=torch.int32, device=device)
    recv = None if payload is None else torch.empty((R, H), dtype=TORCH_DTYPES[payload],
                                                    device=device)
    scales = (torch.empty((R, H // 128), dtype=torch.float32, device=device)
              if payload == "fp8_e4m3" else None)
    return DispatchBuffers(recv, scales, torch.empty(E, **i32), torch.empty(E + 1, **i32),
                           torch.empty(N, **i32), torch.empty(N + 1, **i32),
                           torch.empty(R, **i32), torch.empty(R, **i32))


def alloc_workspace(T: int, E: int, k: int, device="cuda") -> torch.Tensor:
    n = max(moe_dispatch_workspace_bytes(T, E, k), 1)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_dispatch_layout(topk_idx: torch.Tensor, E: int, n_ranks: int, out: DispatchBuffers,
                        workspace: torch.Tensor, stream=None) -> DispatchBuffers:
    T, k = topk_idx.shape
    _debug_check_ids("moe_dispatch_layout", topk_idx, E, stream)
    st = out.as_struct()
    _check("moe_dispatch_layout", load().moe_dispatch_layout(
        _ptr(topk_idx), T, k, E, n_ranks, ctypes.byref(st), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def moe_dispatch_pack(x: torch.Tensor, k: int, token_row: torch.Tensor, recv: torch.Tensor,
                      recv_scales: Optional[torch.Tensor] = None, stream=None):
    T, H = x.shape
    pd = _dtype_code(recv, fp8_ok=True)
    _check("moe_dispatch_pack", load().moe_dispatch_pack(
        _ptr(x), _dtype_code(x), T, H, k, _ptr(token_row), pd, _ptr(recv), _ptr(recv_scales),
        _stream(stream)))
    return recv, recv_scales


def moe_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, E: int, n_ranks: int,
                 out: DispatchBuffers, workspace: torch.Tensor, stream=None) -> DispatchBuffers:
    T, H = x.shape
    k = topk_idx.shape[1]
    _debug_check_ids("moe_dispatch", topk_idx, E, stream)
    st = out.as_struct()
    _check("moe_dispatch", load().moe_dispatch(
        _ptr(x), _dtype_code(x), T, H, _ptr(topk_idx), k, E, n_ranks,
        _dtype_code(out.recv, fp8_ok=True), ctypes.byref(st), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def moe_route_dispatch(logits: torch.Tensor, x: torch.Tensor, k: int, n_ranks: int,
                       out: DispatchBuffers, workspace: torch.Tensor,
                       topk_idx: Optional[torch.Tensor] = None,
                       topk_w: Optional[torch.Tensor] = None, stream=None):
    """Route (top-k ids and weights) and dispatch in one call; returns (topk_idx, topk_w, out)."""
    T, E = logits.shape
    H = x.shape[1]
    assert logits.dtype == torch.float32 and logits.is_contiguous() and x.shape[0] == T
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    st = out.as_struct()
    _check("moe_route_dispatch", load().moe_route_dispatch(
        _ptr(logits), _ptr(x), _dtype_code(x), T, H, E, k, n_ranks,
        _dtype_code(out.recv, fp8_ok=True), _ptr(topk_idx), _ptr(topk_w), ctypes.byref(st),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return topk_idx, topk_w, out


def moe_route_dispatch_noalloc(logits: torch.Tensor, x: torch.Tensor, k: int, n_ranks: int,
                               out: DispatchBuffers, topk_idx: Optional[torch.Tensor] = None,
                               topk_w: Optional[torch.Tensor] = None, stream=None):
    """moe_route_dispatch with the library's fixed device scratch instead of a workspace (the
    call allocates no device memory); returns (topk_idx, topk_w, out)."""
    T, E = logits.shape
    H = x.shape[1]
    assert logits.dtype == torch.float32 and logits.is_contiguous() and x.shape[0] == T
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    st = out.as_struct()
    _check("moe_route_dispatch_noalloc", load().moe_route_dispatch_noalloc(
        _ptr(logits), _ptr(x), _dtype_code(x), T, H, E, k, n_ranks,
        _dtype_code(out.recv, fp8_ok=True), _ptr(topk_idx), _ptr(topk_w), ctypes.byref(st),
        _stream(stream)))
    return topk_idx, topk_w, out


def moe_combine(y: torch.Tensor, token_row: torch.Tensor, topk_w: torch.Tensor,
                out: torch.Tensor, stream=None) -> torch.Tensor:
    T, k = topk_w.shape
    H = y.shape[1]
    _check("moe_combine", load().moe_combine(
        _ptr(y), _dtype_code(y), T, H, k, _ptr(token_row), _ptr(topk_w), _ptr(out),
        _dtype_code(out), _stream(stream)))
    return out


# ------------------------------------------------------------------------------------------------
# Expert parallelism over S sources and N ranks on one GPU (see include/moe_route.h).

def moe_ep_capacity(T: int, E: int, k: int, n_ranks: int) -> int:
    return int(load().moe_ep_capacity(T, E, k, n_ranks))


def moe_ep_send(x: torch.Tensor, topk_idx: torch.Tensor, E: int, n_ranks: int, source: int,
                n_sources: int, cap: int, regions: torch.Tensor, region_counts: torch.Tensor,
                send_row: torch.Tensor, workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """Sender half of dispatch for one source; fills its regions, counts and send_row."""
    T, H = x.shape
    k = topk_idx.shape[1]
    _debug_check_ids("moe_ep_send", topk_idx, E, stream)
    _check("moe_ep_send", load().moe_ep_send(
        _ptr(x), _dtype_code(x), T, H, _ptr(topk_idx), k, E, n_ranks, source, n_sources, cap,
        _ptr(regions), _ptr(region_counts), _ptr(send_row), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return send_row


def moe_ep_recv(regions: torch.Tensor, E: int, n_ranks: int, rank: int, n_sources: int, cap: int,
                region_counts: torch.Tensor, grouped: torch.Tensor, expert_counts: torch.Tensor,
                expert_offsets: torch.Tensor, grouped_src: torch.Tensor, stream=None):
    """Receiver half of dispatch for one rank: grouped rows, counts, offsets, source rows."""
    H = regions.shape[1]
    _check("moe_ep_recv", load().moe_ep_recv(
        _ptr(regions), _dtype_code(regions), H, E, n_ranks, rank, n_sources, cap,
        _ptr(region_counts), _ptr(grouped), _ptr(expert_counts), _ptr(expert_offsets),
        _ptr(grouped_src), _stream(stream)))
    return grouped


def moe_ep_return(y_grouped: torch.Tensor, E: int, n_ranks: int, n_sources: int, cap: int,
                  grouped_src: torch.Tensor, expert_offsets: torch.Tensor, returns: torch.Tensor,
                  stream=None) -> torch.Tensor:
    """Receiver half of combine: expert outputs back to their region rows."""
    H = y_grouped.shape[1]
    _check("moe_ep_return", load().moe_ep_return(
        _ptr(y_grouped), _dtype_code(y_grouped), H, E, n_ranks, n_sources, cap, _ptr(grouped_src),
        _ptr(expert_offsets), _ptr(returns), _stream(stream)))
    return returns


def moe_ep_combine(returns: torch.Tensor, send_row: torch.Tensor, topk_w: torch.Tensor,
                   out: torch.Tensor, stream=None) -> torch.Tensor:
    """Sender half of combine for one source: weighted sum over its returned rows."""
    T, k = topk_w.shape
    H = returns.shape[1]
    _check("moe_ep_combine", load().moe_ep_combine(
        _ptr(returns), _dtype_code(returns), T, H, k, _ptr(send_row), _ptr(topk_w),
        returns.shape[0], _ptr(out), _dtype_code(out), _stream(stream)))
    return out


def moe_ep_partial_rows(topk_idx: torch.Tensor, E: int, n_ranks: int, source: int,
                        n_sources: int, pcap: int, part_row: torch.Tensor,
                        part_counts: torch.Tensor, stream=None) -> torch.Tensor:
    """Partial-row layout of one source: part_row [T, N], part_counts column `source`."""
    T, k = topk_idx.shape
    _check("moe_ep_partial_rows", load().moe_ep_partial_rows(
        _ptr(topk_idx), T, k, E, n_ranks, source, n_sources, pcap, _ptr(part_row),
        _ptr(part_counts), _stream(stream)))
    return part_row


def moe_ep_reduce(y_grouped: torch.Tensor, E: int, n_ranks: int, rank: int, n_sources: int,
                  cap: int, grouped_src: torch.Tensor, topk_idx: torch.Tensor,
                  topk_w: torch.Tensor, send_row: torch.Tensor, part_row: torch.Tensor, pcap: int,
                  partials: torch.Tensor, workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """Expert side of the pre-reduced combine for one rank (source tables stacked)."""
    H = y_grouped.shape[1]
    TT, k = topk_idx.shape
    _check("moe_ep_reduce", load().moe_ep_reduce(
        _ptr(y_grouped), _dtype_code(y_grouped), H, E, n_ranks, rank, n_sources, cap,
        _ptr(grouped_src), TT // n_sources, k, _ptr(topk_idx), _ptr(topk_w), _ptr(send_row),
        _ptr(part_row), pcap, _ptr(partials), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return partials


def moe_ep_reduce_workspace(n_sources: int, cap: int, device="cuda") -> torch.Tensor:
    n = max(int(load().moe_ep_reduce_workspace_bytes(n_sources, cap)), 1)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_ep_combine_reduced(partials: torch.Tensor, part_row: torch.Tensor, out: torch.Tensor,
                           stream=None) -> torch.Tensor:
    """Source side of the pre-reduced combine: a token's partial rows added in rank order."""
    T, N = part_row.shape
    H = partials.shape[1]
    _check("moe_ep_combine_reduced", load().moe_ep_combine_reduced(
        _ptr(partials), _dtype_code(partials), T, H, N, _ptr(part_row), partials.shape[0],
        _ptr(out), _dtype_code(out), _stream(stream)))
    return out
