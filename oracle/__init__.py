"""CPU oracle for MoE top-k routing, dispatch and combine (ctypes wrapper over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` are the only callers. The HIP path never imports this package, and this package never
imports the HIP path; they share only the seeded input generators.

Arrays are numpy: f32 as float32, bf16 as uint16 bit patterns, fp8-e4m3 as uint8 codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
# Tests may point the wrapper at another build of the same source (planted-mistake checks).
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")

DTYPES = {"f32": 0, "bf16": 1, "fp8_e4m3": 2}
NP_DTYPES = {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}
EXPERT_RULES = {"identity": 0, "scale": 1}

_lib = None


def build() -> str:
    """Compile the oracle with gcc: -O2, no fast-math, no FMA contraction."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
                           "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
        P, I, L = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        for name, args in {
            "oracle_f32_to_bf16": [P, P, L], "oracle_f64_to_bf16": [P, P, L],
            "oracle_f32_to_e4m3": [P, P, L], "oracle_e4m3_to_f32": [P, P, L],
            "oracle_route": [P, I, I, I, P, P],
            "oracle_dispatch": [P, I, I, I, P, I, I, I, I, P, P, P, P, P, P, P, P],
            "oracle_experts": [P, I, P, I, I, P, I, I, P, I],
            "oracle_combine": [P, I, I, I, I, P, P, P, I],
            "oracle_ep_send": [P, I, I, I, P, I, I, I, I, I, I, P, P, P],
            "oracle_ep_recv": [P, I, I, I, I, I, I, I, P, P, P, P, P],
            "oracle_ep_return": [P, I, I, L, P, P],
            "oracle_ep_partial_rows": [P, I, I, I, I, I, I, I, P, P],
            "oracle_ep_reduce": [P, I, I, I, I, I, I, I, P, I, I, P, P, P, P, P],
            "oracle_ep_combine_reduced": [P, I, I, I, I, P, P, I],
            "oracle_check_topk": [P, I, I, I, P],
        }.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = None if name.startswith("oracle_f") or name.startswith("oracle_e4") else I
        _lib = lib
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f32_to_bf16(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().oracle_f32_to_bf16(_p(a), _p(out), a.size)
    return out


def f64_to_bf16(a) -> np.ndarray:
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().oracle_f64_to_bf16(_p(a), _p(out), a.size)
    return out


def f32_to_e4m3(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().oracle_f32_to_e4m3(_p(a), _p(out), a.size)
    return out


def e4m3_to_f32(a) -> np.ndarray:
    a = _c(a, np.uint8)
    out = np.empty(a.shape, np.float32)
    _load().oracle_e4m3_to_f32(_p(a), _p(out), a.size)
    return out


def bf16_to_f32(a) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    return (_c(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def route(logits, k: int):
    """Top-k experts per token (largest logit first, ties to the lower id) and renormalised
    softmax weights. Returns (topk_idx int32 [T,k], topk_w float32 [T,k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = _load().oracle_route(_p(logits), T, E, k, _p(idx), _p(w))
    if rc:
        raise ValueError(f"oracle_route rejected its arguments (code {rc})")
    return idx, w


def dispatch(x, x_dtype: str, topk_idx, E: int, N: int, payload: str) -> dict:
    """Counts, offsets, row maps and the packed receive buffer, all as numpy arrays."""
    x = _c(x, NP_DTYPES[x_dtype])
    topk_idx = _c(topk_idx, np.int32)
    T, H = x.shape
    k = topk_idx.shape[1]
    R = T * k
    out = {
        "recv": np.empty((R, H), NP_DTYPES[payload]),
        "recv_scales": np.empty((R, H // 128), np.float32) if payload == "fp8_e4m3" else None,
        "expert_counts": np.empty(E, np.int32), "expert_offsets": np.empty(E + 1, np.int32),
        "rank_counts": np.empty(N, np.int32), "rank_offsets": np.empty(N + 1, np.int32),
        "token_row": np.empty(R, np.int32), "row_token": np.empty(R, np.int32),
    }
    rc = _load().oracle_dispatch(
        _p(x), DTYPES[x_dtype], T, H, _p(topk_idx), k, E, N, DTYPES[payload], _p(out["recv"]),
        _p(out["recv_scales"]), _p(out["expert_counts"]), _p(out["expert_offsets"]),
        _p(out["rank_counts"]), _p(out["rank_offsets"]), _p(out["token_row"]),
        _p(out["row_token"]))
    if rc:
        raise ValueError(f"oracle_dispatch rejected its arguments (code {rc})")
    return out


def experts(recv, payload: str, recv_scales, expert_offsets, rule: str, y_dtype: str) -> np.ndarray:
    """Emulated expert outputs y [R,H] (identity, or row * (expert+1)/256)."""
    recv = _c(recv, NP_DTYPES[payload])
    R, H = recv.shape
    E = len(expert_offsets) - 1
    scales = None if recv_scales is None else _c(recv_scales, np.float32)
    offs = _c(expert_offsets, np.int32)
    y = np.empty((R, H), NP_DTYPES[y_dtype])
    rc = _load().oracle_experts(_p(recv), DTYPES[payload], _p(scales), R, H, _p(offs), E,
                                EXPERT_RULES[rule], _p(y), DTYPES[y_dtype])
    if rc:
        raise ValueError(f"oracle_experts rejected its arguments (code {rc})")
    return y


def combine(y, y_dtype: str, token_row, topk_w, out_dtype: str) -> np.ndarray:
    """out[t] = sum_j w[t,j] * y[token_row[t*k+j]] in double, rounded once to out_dtype."""
    y = _c(y, NP_DTYPES[y_dtype])
    topk_w = _c(topk_w, np.float32)
    token_row = _c(token_row, np.int32).reshape(-1)
    T, k = topk_w.shape
    H = y.shape[1]
    out = np.empty((T, H), NP_DTYPES[out_dtype])
    rc = _load().oracle_combine(_p(y), DTYPES[y_dtype], T, H, k, _p(token_row), _p(topk_w),
                                _p(out), DTYPES[out_dtype])
    if rc:
        raise ValueError(f"oracle_combine rejected its arguments (code {rc})")
    return out


# ------------------------------------------------------------------------------------------------
# Expert parallelism over S sources and N ranks, emulated on one device: the region array holds
# one region of `cap` rows per (rank r, source s), at rows [(r*S + s)*cap, (r*S + s + 1)*cap).

def ep_capacity(T: int, E: int, k: int, N: int) -> int:
    """Rows of one (rank, source) region: the most one source can send to one rank."""
    return T * min(k, E // N)


def ep_send(x, x_dtype: str, topk_idx, E: int, N: int, source: int, S: int, cap: int, regions,
            region_counts) -> np.ndarray:
    """Sender half of dispatch for one source: writes its rows into `regions` [N*S*cap, H] and its
    counts into `region_counts` [N, S, E/N] (both in place); returns send_row int32 [T*k]."""
    x = _c(x, NP_DTYPES[x_dtype])
    topk_idx = _c(topk_idx, np.int32)
    T, H = x.shape
    k = topk_idx.shape[1]
    assert regions.flags.c_contiguous and regions.shape == (N * S * cap, H)
    assert region_counts.flags.c_contiguous and region_counts.dtype == np.int32
    send_row = np.empty(T * k, np.int32)
    rc = _load().oracle_ep_send(_p(x), DTYPES[x_dtype], T, H, _p(topk_idx), k, E, N, source, S,
                                cap, _p(regions), _p(region_counts), _p(send_row))
    if rc:
        raise ValueError(f"oracle_ep_send rejected its arguments (code {rc})")
    return send_row


def ep_recv(regions, dtype: str, E: int, N: int, rank: int, S: int, cap: int,
            region_counts) -> dict:
    """Receiver half of dispatch for one rank: grouped rows [S*cap, H] ordered by (local expert,
    source, token, slot), per-expert counts and offsets, and each grouped row's region row."""
    regions = _c(regions, NP_DTYPES[dtype])
    H = regions.shape[1]
    L = E // N
    out = {"grouped": np.zeros((S * cap, H), NP_DTYPES[dtype]),
           "expert_counts": np.empty(L, np.int32), "expert_offsets": np.empty(L + 1, np.int32),
           "grouped_src": np.empty(S * cap, np.int32)}
    rc = _load().oracle_ep_recv(_p(regions), DTYPES[dtype], H, E, N, rank, S, cap,
                                _p(_c(region_counts, np.int32)), _p(out["grouped"]),
                                _p(out["expert_counts"]), _p(out["expert_offsets"]),
                                _p(out["grouped_src"]))
    if rc:
        raise ValueError(f"oracle_ep_recv rejected its arguments (code {rc})")
    return out


def ep_return(y_grouped, dtype: str, grouped_src, returns) -> None:
    """Receiver half of combine: returns[grouped_src[g]] = y_grouped[g] for every valid g."""
    y_grouped = _c(y_grouped, NP_DTYPES[dtype])
    assert returns.flags.c_contiguous and returns.dtype == NP_DTYPES[dtype]
    n, H = y_grouped.shape
    rc = _load().oracle_ep_return(_p(y_grouped), DTYPES[dtype], H, n,
                                  _p(_c(grouped_src, np.int32)), _p(returns))
    if rc:
        raise ValueError(f"oracle_ep_return rejected its arguments (code {rc})")


# Combine with pre-reduction on the expert side: rank r sends one partial row per (token, rank),
# the source adds the partial rows of each token.

def ep_partial_rows(topk_idx, E: int, N: int, source: int, S: int, pcap: int, part_counts):
    """part_row int32 [T, N] (partial-array row of (token, rank), -1 if the token has no expert
    on the rank); fills part_counts [N, S] column `source` in place."""
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    part_row = np.empty((T, N), np.int32)
    assert part_counts.flags.c_contiguous and part_counts.dtype == np.int32
    rc = _load().oracle_ep_partial_rows(_p(topk_idx), T, k, E, N, source, S, pcap, _p(part_row),
                                        _p(part_counts))
    if rc:
        raise ValueError(f"oracle_ep_partial_rows rejected its arguments (code {rc})")
    return part_row


def ep_reduce(y_grouped, dtype: str, E: int, N: int, rank: int, S: int, cap: int, grouped_src,
              topk_idx, topk_w, send_row, part_row, partials) -> None:
    """Partial rows of one rank for all sources, written into `partials` in place. The source
    tables are stacked: source s owns tokens [s*T, (s+1)*T)."""
    y_grouped = _c(y_grouped, NP_DTYPES[dtype])
    topk_idx = _c(topk_idx, np.int32)
    TT, k = topk_idx.shape
    T = TT // S
    H = y_grouped.shape[1]
    assert partials.flags.c_contiguous and partials.dtype == NP_DTYPES[dtype]
    rc = _load().oracle_ep_reduce(
        _p(y_grouped), DTYPES[dtype], H, E, N, rank, S, cap, _p(_c(grouped_src, np.int32)), T, k,
        _p(topk_idx), _p(_c(topk_w, np.float32)), _p(_c(send_row, np.int32)),
        _p(_c(part_row, np.int32)), _p(partials))
    if rc:
        raise ValueError(f"oracle_ep_reduce rejected its arguments (code {rc})")


def ep_combine_reduced(partials, dtype: str, part_row, out_dtype: str) -> np.ndarray:
    """out[t] = sum over ranks of the token's partial rows, rounded once."""
    partials = _c(partials, NP_DTYPES[dtype])
    part_row = _c(part_row, np.int32)
    T, N = part_row.shape
    H = partials.shape[1]
    out = np.empty((T, H), NP_DTYPES[out_dtype])
    rc = _load().oracle_ep_combine_reduced(_p(partials), DTYPES[dtype], T, H, N, _p(part_row),
                                           _p(out), DTYPES[out_dtype])
    if rc:
        raise ValueError(f"oracle_ep_combine_reduced rejected its arguments (code {rc})")
    return out


def check_topk(topk_idx, E: int) -> tuple:
    """(ids outside [0, E), in-range ids repeating an earlier slot of their token)."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    counts = np.zeros(2, np.int64)
    assert _load().oracle_check_topk(_p(idx), T, k, E, _p(counts)) == 0
    return int(counts[0]), int(counts[1])
