"""CPU oracle for MoE expert-parallel dispatch/combine (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. It wraps the plain C loops of ``ep_oracle.c`` with
ctypes and numpy array plumbing; every step of the arithmetic is in C.
It shares no code with the HIP library and never imports it.

Method source: "Enabling trillion-parameter models on AWS EFA" (Perplexity),
sections "Send and receive buffers" and "Dispatch and combine".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

STATUS_BAD_EXPERT = 1
STATUS_CAPACITY = 2

_lib = None


def build() -> str:
    """Compile the oracle with gcc: plain C, -O2, no vector intrinsics."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def _declare(L: ctypes.CDLL) -> None:
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_f32.restype = ctypes.c_float
    L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    L.oracle_f64_to_bf16.restype = ctypes.c_uint16
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_to_f32.restype = ctypes.c_float
    L.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    L.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    L.oracle_quantize_b128.argtypes = [_I, _P, _P, _P]
    L.oracle_quantize_b128.restype = None
    L.oracle_dispatch_pack_quant.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
    L.oracle_dispatch_pack_quant.restype = None
    L.oracle_recv_bound.argtypes = [_I, _I, _I, _I]
    L.oracle_recv_bound.restype = _I64
    L.oracle_plan.argtypes = [_I, _I, _I, _I, _I64] + [_P] * 8
    L.oracle_plan.restype = _I
    L.oracle_dispatch_pack.argtypes = [_I, _I, _I, _I64, _P, _P, _P]
    L.oracle_dispatch_pack.restype = None
    L.oracle_transfer.argtypes = [_I, _I, _I, _I, _I64, _I64, _P, _P, _P, _P]
    L.oracle_transfer.restype = None
    L.oracle_unpack.argtypes = [_I, _I, _I, _I, _I64, _I64, _I64] + [_P] * 6
    L.oracle_unpack.restype = None
    L.oracle_expert_bf16.argtypes = [_I, _P, _P, _I, _P]
    L.oracle_expert_bf16.restype = None
    L.oracle_expert_fp8.argtypes = [_I, _P, _P, _P]
    L.oracle_expert_fp8.restype = None
    L.oracle_expert_op.argtypes = [_I, _I, _I, _I64, _I, _P, _P, _P, _P, _P]
    L.oracle_expert_op.restype = None
    L.oracle_combine_token.argtypes = [_I, _I, _P, _P, _P]
    L.oracle_combine_token.restype = None
    L.oracle_combine.argtypes = [_I, _I, _I, _I, _I, _I64, _P, _P, _P, _P, _P]
    L.oracle_combine.restype = None
    L.oracle_combine_presum_token.argtypes = [_I, _I, _P, _P, _P, _P, _P]
    L.oracle_combine_presum_token.restype = None
    L.oracle_combine_presum.argtypes = [_I, _I, _I, _I, _I, _I64] + [_P] * 6
    L.oracle_combine_presum.restype = None
    L.oracle_kv_regions.argtypes = [_I64, _I64, _I64, _P, _I64, _P, _P, _P, _P]
    L.oracle_kv_regions.restype = _I64
    L.oracle_kv_copy.argtypes = [_I, _I64, _P, _P, _P, _P, _I64, _P, _I64]
    L.oracle_kv_copy.restype = None
    L.oracle_rounding_mode_is_nearest.argtypes = []
    L.oracle_rounding_mode_is_nearest.restype = _I


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# Scalar codecs (for pins and sampled checks)
# ---------------------------------------------------------------------------

def f64_to_bf16(v: float) -> int:
    return int(lib().oracle_f64_to_bf16(float(v)))


def f32_to_bf16(v: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(v)))


def bf16_to_f32(b: int) -> float:
    return float(lib().oracle_bf16_to_f32(int(b)))


def e4m3_to_f32(c: int) -> float:
    return float(lib().oracle_e4m3_to_f32(int(c)))


def f32_to_e4m3(v: float) -> int:
    return int(lib().oracle_f32_to_e4m3(float(v)))


def quantize_b128(x_bf16: np.ndarray):
    """bf16 rows [..., H] -> (e4m3 codes uint8 [..., H], scales fp32 [..., H/128])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    H = x.shape[-1]
    rows = x.reshape(-1, H)
    codes = np.zeros(rows.shape, np.uint8)
    scales = np.zeros((rows.shape[0], H // 128), np.float32)
    for i in range(rows.shape[0]):
        lib().oracle_quantize_b128(H, _ptr(rows[i]), _ptr(codes[i]), _ptr(scales[i]))
    return codes.reshape(x.shape), scales.reshape(*x.shape[:-1], H // 128)


def dispatch_pack_quant(x_bf16: np.ndarray, p: dict):
    """bf16 x [N, T, H] -> fp8 send planes (codes [N, T*R, H], scales [N, T*R, H/128])."""
    N, T, H = x_bf16.shape
    R = p["send_pos"].shape[2]
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    codes = np.zeros((N, T * R, H), np.uint8)
    scales = np.zeros((N, T * R, H // 128), np.float32)
    lib().oracle_dispatch_pack_quant(N, T, R, H, _ptr(x), _ptr(p["send_pos"]), _ptr(codes),
                                     _ptr(scales))
    return codes, scales


def recv_bound(N: int, T: int, E: int, R: int) -> int:
    return int(lib().oracle_recv_bound(N, T, E, R))


# ---------------------------------------------------------------------------
# Plan
# ---------------------------------------------------------------------------

def plan(N: int, T: int, E: int, R: int, cap: int, idx: np.ndarray) -> dict:
    """Counts, send offsets/positions, receive and grouped offsets/positions."""
    L = E // N
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(N, T, R)
    out = {
        "cnt": np.zeros((N, E), np.int32),
        "send_off": np.zeros((N, E + 1), np.int32),
        "send_pos": np.zeros((N, T, R), np.int32),
        "recv_off": np.zeros((N, N + 1), np.int32),
        "grp_off": np.zeros((N, L + 1), np.int32),
        "grp_pos": np.zeros((N, T, R), np.int32),
    }
    st = np.zeros(1, np.int32)
    rc = lib().oracle_plan(N, T, E, R, int(cap), _ptr(idx), _ptr(out["cnt"]),
                           _ptr(out["send_off"]), _ptr(out["send_pos"]),
                           _ptr(out["recv_off"]), _ptr(out["grp_off"]),
                           _ptr(out["grp_pos"]), _ptr(st))
    if rc != 0:
        raise ValueError(f"oracle_plan rejected the shape (rc={rc})")
    out["status"] = int(st[0])
    return out


# ---------------------------------------------------------------------------
# Payload
# ---------------------------------------------------------------------------

def dispatch_pack(plane: np.ndarray, p: dict) -> np.ndarray:
    """plane: uint8 [N, T, row] -> send plane uint8 [N, T*R, row]."""
    N, T, row = plane.shape
    R = p["send_pos"].shape[2]
    plane = np.ascontiguousarray(plane)
    send = np.zeros((N, T * R, row), np.uint8)
    lib().oracle_dispatch_pack(N, T, R, row, _ptr(plane), _ptr(p["send_pos"]), _ptr(send))
    return send


def transfer(send: np.ndarray, p: dict, recv_rows: int) -> np.ndarray:
    """send [N, T*R, row] -> receive buffers [N, recv_rows, row]."""
    N, TR, row = send.shape
    E = p["cnt"].shape[1]
    T, R = p["send_pos"].shape[1:]
    recv = np.zeros((N, recv_rows, row), np.uint8)
    lib().oracle_transfer(N, T, E, R, row, recv_rows, _ptr(send),
                          _ptr(p["send_off"]), _ptr(p["recv_off"]), _ptr(recv))
    return recv


def unpack(recv: np.ndarray, p: dict, rows: int, fill: int = 0) -> np.ndarray:
    """receive buffers [N, recv_rows, row] -> grouped [N, rows, row]; rows
    the unpack does not write keep the byte `fill`."""
    N, recv_rows, row = recv.shape
    E = p["cnt"].shape[1]
    T, R = p["send_pos"].shape[1:]
    grouped = np.full((N, rows, row), fill, np.uint8)
    lib().oracle_unpack(N, T, E, R, row, recv_rows, rows, _ptr(recv),
                        _ptr(p["cnt"]), _ptr(p["send_off"]), _ptr(p["recv_off"]),
                        _ptr(p["grp_off"]), _ptr(grouped))
    return grouped


def expert_op(grouped: list, p: dict, H: int, payload: int,
              alpha: Optional[np.ndarray]) -> np.ndarray:
    """Stand-in expert on grouped planes -> bf16 bits [N, rows, H]."""
    N, rows, _ = grouped[0].shape
    E = p["cnt"].shape[1]
    y = np.zeros((N, rows, H), np.uint16)
    g0 = np.ascontiguousarray(grouped[0])
    g1 = np.ascontiguousarray(grouped[1]) if payload == 1 else None
    a = np.ascontiguousarray(alpha, dtype=np.float32) if alpha is not None else None
    lib().oracle_expert_op(N, E, H, rows, payload, _ptr(g0), _ptr(g1), _ptr(a),
                           _ptr(p["grp_off"]), _ptr(y))
    return y


def combine(y: np.ndarray, weights: np.ndarray, idx: np.ndarray, p: dict) -> np.ndarray:
    """Expert outputs bf16 [N, rows, H] -> combined tokens bf16 [N, T, H]."""
    N, rows, H = y.shape
    T, R = idx.shape[1:]
    E = p["cnt"].shape[1]
    out = np.zeros((N, T, H), np.uint16)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    lib().oracle_combine(N, T, E, R, H, rows, _ptr(idx), _ptr(p["grp_pos"]),
                         _ptr(np.ascontiguousarray(y)), _ptr(w), _ptr(out))
    return out


def combine_token(w: np.ndarray, rows: list) -> np.ndarray:
    """One token from explicit expert rows (None = dropped slot)."""
    R = len(rows)
    H = next(r.shape[0] for r in rows if r is not None) if any(r is not None for r in rows) else 0
    keep = [np.ascontiguousarray(r, dtype=np.uint16) if r is not None else None for r in rows]
    arr = (ctypes.c_void_p * R)(*[(r.ctypes.data if r is not None else None) for r in keep])
    out = np.zeros(H, np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    lib().oracle_combine_token(H, R, _ptr(w), ctypes.cast(arr, ctypes.c_void_p), _ptr(out))
    return out


def combine_presum(y: np.ndarray, weights: np.ndarray, idx: np.ndarray, p: dict):
    """Partial sums on the expert side, then on the source side.
    Returns (partial bf16 [N, T*R, H] with leader rows set (others 0),
    out bf16 [N, T, H])."""
    N, rows, H = y.shape
    T, R = idx.shape[1:]
    E = p["cnt"].shape[1]
    partial = np.zeros((N, T * R, H), np.uint16)
    out = np.zeros((N, T, H), np.uint16)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    lib().oracle_combine_presum(N, T, E, R, H, rows, _ptr(idx), _ptr(p["grp_pos"]),
                                _ptr(np.ascontiguousarray(y)), _ptr(w), _ptr(partial), _ptr(out))
    return partial, out


def combine_presum_token(w: np.ndarray, rows: list, ranks: list) -> np.ndarray:
    """One token of the partial-sum combine from explicit expert rows and the
    ranks hosting them (None = dropped slot)."""
    R = len(rows)
    H = next(r.shape[0] for r in rows if r is not None) if any(r is not None for r in rows) else 0
    keep = [np.ascontiguousarray(r, dtype=np.uint16) if r is not None else None for r in rows]
    arr = (ctypes.c_void_p * R)(*[(r.ctypes.data if r is not None else None) for r in keep])
    rk = np.array([-1 if r is None else int(r) for r in ranks], np.int32)
    partial = np.zeros((max(R, 1), max(H, 1)), np.uint16)
    out = np.zeros(H, np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    lib().oracle_combine_presum_token(H, R, _ptr(w), ctypes.cast(arr, ctypes.c_void_p), _ptr(rk),
                                      _ptr(partial), _ptr(out))
    return out


def kv_regions(n: int, tok: int, bs_src: int, src_blocks: np.ndarray, bs_dst: int,
               dst_blocks: np.ndarray) -> np.ndarray:
    """Transfer regions of one request: int64 [m, 3] rows (src_off, dst_off, bytes)."""
    sb = np.ascontiguousarray(src_blocks, dtype=np.int32)
    db = np.ascontiguousarray(dst_blocks, dtype=np.int32)
    so = np.zeros(max(n, 1), np.int64)
    do = np.zeros(max(n, 1), np.int64)
    by = np.zeros(max(n, 1), np.int64)
    m = lib().oracle_kv_regions(n, tok, bs_src, _ptr(sb), bs_dst, _ptr(db), _ptr(so), _ptr(do),
                                _ptr(by))
    return np.stack([so[:m], do[:m], by[:m]], axis=1)


def kv_copy(regions: np.ndarray, src: np.ndarray, dst: np.ndarray) -> np.ndarray:
    """Apply regions to every rank: src uint8 [ranks, src_bytes], dst uint8
    [ranks, dst_bytes] (a copy of dst is returned)."""
    out = np.ascontiguousarray(dst).copy()
    src = np.ascontiguousarray(src)
    reg = np.ascontiguousarray(regions, dtype=np.int64)
    so, do, by = (np.ascontiguousarray(reg[:, c]) for c in range(3))
    lib().oracle_kv_copy(src.shape[0], reg.shape[0], _ptr(so), _ptr(do), _ptr(by), _ptr(src),
                         src.shape[1], _ptr(out), out.shape[1])
    return out


def expert_row(row_planes: list, e: int, payload: int, H: int,
               alpha: Optional[np.ndarray]) -> np.ndarray:
    """Stand-in expert applied to one token row (payload planes of one row)."""
    out = np.zeros(H, np.uint16)
    if payload == 0:
        inp = np.ascontiguousarray(row_planes[0]).view(np.uint16)
        a = np.ascontiguousarray(alpha, dtype=np.float32) if alpha is not None else None
        lib().oracle_expert_bf16(H, _ptr(inp), _ptr(a), int(e), _ptr(out))
    else:
        codes = np.ascontiguousarray(row_planes[0])
        scales = np.ascontiguousarray(row_planes[1]).view(np.float32)
        lib().oracle_expert_fp8(H, _ptr(codes), _ptr(scales), _ptr(out))
    return out


# ---------------------------------------------------------------------------
# Whole path
# ---------------------------------------------------------------------------

def run(wl, cap: Optional[int] = None, with_payload: bool = True) -> dict:
    """Plan, pack, transfer, unpack, expert, combine for one workload.

    Buffers hold min(cap, largest delivered count) rows per destination;
    rows at or beyond that are never defined, so nothing is lost.
    """
    sh = wl.shape
    N, T, H, E, R = sh.n_ranks, sh.tokens, sh.hidden, sh.n_experts, sh.topk
    if cap is None:
        cap = sh.cap_rows if sh.cap_rows > 0 else recv_bound(N, T, E, R)
    p = plan(N, T, E, R, cap, wl.idx)
    res = {"plan": p, "cap": cap}
    if not with_payload:
        return res
    totals = p["recv_off"][:, N]
    rows = int(max(1, min(cap, int(totals.max()) if N else 0)))
    recv_rows = int(max(1, int(totals.max())))
    send, recv, grouped = [], [], []
    for plane in wl.planes:
        s = dispatch_pack(plane, p)
        r = transfer(s, p, recv_rows)
        g = unpack(r, p, rows)
        send.append(s)
        recv.append(r)
        grouped.append(g)
    y = expert_op(grouped, p, H, sh.payload, wl.alpha)
    out = combine(y, wl.weights, wl.idx, p)
    res.update(send=send, recv=recv, grouped=grouped, y=y, out=out, rows=rows)
    return res
