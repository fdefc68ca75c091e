"""Python binding of the gfx950 MoE expert-parallel dispatch/combine library.

Thin ctypes layer over the C ABI in ``include/ep.h``: the functions below
have the same names as the C entry points and only marshal arguments
(tensor data pointers, the current HIP stream). Every step of the path runs
in the library's HIP kernels; there is no fallback. If the compiled library
is missing, importing this package raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libep_mi355x.so")

EP_OK = 0
EP_ERR_INVALID_ARG = -1
EP_ERR_UNSUPPORTED = -2
EP_ERR_DEVICE_MISMATCH = -3
EP_ERR_HIP = -4
EP_STATUS_BAD_EXPERT = 1
EP_STATUS_CAPACITY = 2
EP_STATUS_BAD_REGION = 4
EP_PAYLOAD_BF16 = 0
EP_PAYLOAD_FP8_B128 = 1
EP_KV_STATIC_SLOTS = 64
EP_PROBE_COPY, EP_PROBE_FILL, EP_PROBE_READ, EP_PROBE_SCATTER, EP_PROBE_SCATTER_WIDE = range(5)
EP_PROBE_NT_LOADS, EP_PROBE_XCD, EP_PROBE_ONE_WAVE = 1, 2, 4

# Every entry point the C header declares (checked by the tests).
EXPORTS = (
    "ep_recv_bound", "ep_capacity", "ep_num_planes", "ep_row_bytes",
    "ep_plan_bytes", "ep_plan_views", "ep_plan", "ep_dispatch", "ep_dispatch_quant",
    "ep_dispatch_pack",
    "ep_dispatch_pack_quant",
    "ep_dispatch_transfer", "ep_dispatch_unpack", "ep_dispatch_recv",
    "ep_dispatch_send", "ep_dispatch_recv_split", "ep_dispatch_send_plan",
    "ep_dispatch_send_pack", "ep_dispatch_recv_plan", "ep_dispatch_recv_pull",
    "ep_expert_stub", "ep_combine",
    "ep_combine_presum", "ep_kv_plan", "ep_kv_push", "ep_kv_push_staged",
    "ep_kv_push_staged_static",
    "ep_probe_copy", "ep_probe_pattern", "ep_status_string",
    "ep_last_error",
)


class EPError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where} failed ({code}): {msg}")
        self.code = code


class Desc(ctypes.Structure):
    """ep_desc: N, T, H, E, R, payload, cap_rows (0 = worst-case bound)."""
    _fields_ = [
        ("n_ranks", ctypes.c_int32), ("tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("payload", ctypes.c_int32),
        ("cap_rows", ctypes.c_int64),
    ]


class PlanView(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "cnt", "send_off", "send_pos", "recv_off", "grp_off", "grp_pos",
        "src_off", "comb_row", "grp_slot", "send_slot", "recv_rows", "send_seg", "win_list")]


def _load() -> ctypes.CDLL:
    # torch first: it loads its own HIP runtime, and the library's dependency
    # on libamdhip64.so.7 must resolve to that same, already-loaded copy
    # (two HIP runtimes in one process would not share devices or memory).
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, D, I64 = ctypes.c_void_p, ctypes.POINTER(Desc), ctypes.c_int64
    sig = {
        "ep_recv_bound": (ctypes.c_int64, [D]),
        "ep_capacity": (ctypes.c_int64, [D]),
        "ep_num_planes": (ctypes.c_int, [D]),
        "ep_row_bytes": (ctypes.c_int64, [D, ctypes.c_int]),
        "ep_plan_bytes": (ctypes.c_size_t, [D]),
        "ep_plan_views": (ctypes.c_int, [D, P, ctypes.POINTER(PlanView)]),
        "ep_plan": (ctypes.c_int, [D, P, P, P, P]),
        "ep_dispatch": (ctypes.c_int, [D, P, P, P, P, P, P, P]),
        "ep_dispatch_quant": (ctypes.c_int, [D, P, P, P, P, P, P, P]),
        "ep_dispatch_pack": (ctypes.c_int, [D, P, P, P, P]),
        "ep_dispatch_pack_quant": (ctypes.c_int, [D, P, P, P, P]),
        "ep_dispatch_transfer": (ctypes.c_int, [D, P, P, P, P]),
        "ep_dispatch_unpack": (ctypes.c_int, [D, P, P, P, P]),
        "ep_dispatch_recv": (ctypes.c_int, [D, P, P, P, P]),
        "ep_dispatch_send": (ctypes.c_int, [D, P, P, P, P, P, ctypes.c_int32, P, P]),
        "ep_dispatch_recv_split": (ctypes.c_int, [D, P, P, ctypes.c_int32, P, P, P, P]),
        "ep_dispatch_send_plan": (ctypes.c_int, [D, P, P, P, P]),
        "ep_dispatch_send_pack": (ctypes.c_int, [D, P, P, P, P, P, ctypes.c_int32, P]),
        "ep_dispatch_recv_plan": (ctypes.c_int, [D, P, P, P]),
        "ep_dispatch_recv_pull": (ctypes.c_int, [D, P, P, ctypes.c_int32, P, P, P]),
        "ep_expert_stub": (ctypes.c_int, [D, P, P, P, P, P]),
        "ep_combine": (ctypes.c_int, [D, P, P, P, P, P]),
        "ep_combine_presum": (ctypes.c_int, [D, P, P, P, P, P, P]),
        "ep_kv_plan": (ctypes.c_int64, [I64, I64, I64, P, I64, P, ctypes.c_int32, P, I64]),
        "ep_kv_push": (ctypes.c_int, [ctypes.c_int32, P, I64, I64, P, I64, P, I64, P, P, P]),
        "ep_kv_push_staged": (ctypes.c_int, [ctypes.c_int32, P, I64, I64, P, I64, P, I64, P,
                                             ctypes.c_int32, P, P, P]),
        "ep_kv_push_staged_static": (ctypes.c_int, [ctypes.c_int32, P, I64, I64, P, I64, P, I64,
                                                    ctypes.c_int32, P, P, P]),
        "ep_probe_copy": (ctypes.c_int, [P, P, ctypes.c_size_t, P]),
        "ep_probe_pattern": (ctypes.c_int, [P, P, P, I64, I64, I64, I64, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int, I64, P]),
        "ep_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "ep_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


# ---------------------------------------------------------------------------
# Marshalling helpers
# ---------------------------------------------------------------------------

def make_desc(n_ranks, tokens, hidden, n_experts, topk,
              payload=EP_PAYLOAD_BF16, cap_rows=0) -> Desc:
    return Desc(n_ranks, tokens, hidden, n_experts, topk, payload, cap_rows)


def _addr(t) -> Optional[int]:
    """Address of a buffer: None, a raw device address, or a tensor, which
    must be contiguous (the library reads every buffer as dense row-major
    bytes; a strided view would be read as if it were dense)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError(f"buffer of shape {tuple(t.shape)} and strides {t.stride()} is not "
                         "contiguous: the library takes dense row-major buffers")
    return t.data_ptr()


def _planes(ts: Sequence) -> ctypes.Array:
    ts = list(ts) + [None] * (2 - len(ts))
    return (ctypes.c_void_p * 2)(*[_addr(t) for t in ts[:2]])


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> int:
    if rc != EP_OK:
        raise EPError(rc, where, _lib.ep_last_error().decode())
    return rc


def status_string(code: int) -> str:
    return _lib.ep_status_string(code).decode()


def last_error() -> str:
    return _lib.ep_last_error().decode()


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def recv_bound(d: Desc) -> int:
    return int(_lib.ep_recv_bound(ctypes.byref(d)))


def capacity(d: Desc) -> int:
    return int(_lib.ep_capacity(ctypes.byref(d)))


def num_planes(d: Desc) -> int:
    return int(_lib.ep_num_planes(ctypes.byref(d)))


def row_bytes(d: Desc, plane: int) -> int:
    return int(_lib.ep_row_bytes(ctypes.byref(d), plane))


def plan_bytes(d: Desc) -> int:
    return int(_lib.ep_plan_bytes(ctypes.byref(d)))


def plan_views(d: Desc, plan_ws) -> PlanView:
    v = PlanView()
    _check(_lib.ep_plan_views(ctypes.byref(d), _addr(plan_ws), ctypes.byref(v)), "ep_plan_views")
    return v


def plan(d: Desc, topk_idx, plan_ws, status, stream=None) -> None:
    _check(_lib.ep_plan(ctypes.byref(d), _addr(topk_idx), _addr(plan_ws), _addr(status),
                        _stream(stream)), "ep_plan")


def dispatch(d: Desc, topk_idx, x: Sequence, plan_ws, send: Sequence, grouped: Sequence, status,
             stream=None) -> None:
    _check(_lib.ep_dispatch(ctypes.byref(d), _addr(topk_idx), _planes(x), _addr(plan_ws),
                            _planes(send), _planes(grouped), _addr(status), _stream(stream)),
           "ep_dispatch")


def dispatch_quant(d: Desc, topk_idx, x_bf16, plan_ws, send: Sequence, grouped: Sequence, status,
                   stream=None) -> None:
    _check(_lib.ep_dispatch_quant(ctypes.byref(d), _addr(topk_idx), _addr(x_bf16), _addr(plan_ws),
                                  _planes(send), _planes(grouped), _addr(status), _stream(stream)),
           "ep_dispatch_quant")


def dispatch_pack(d: Desc, x: Sequence, plan_ws, send: Sequence, stream=None) -> None:
    _check(_lib.ep_dispatch_pack(ctypes.byref(d), _planes(x), _addr(plan_ws), _planes(send),
                                 _stream(stream)), "ep_dispatch_pack")


def dispatch_pack_quant(d: Desc, x_bf16, plan_ws, send: Sequence, stream=None) -> None:
    _check(_lib.ep_dispatch_pack_quant(ctypes.byref(d), _addr(x_bf16), _addr(plan_ws), _planes(send),
                                       _stream(stream)), "ep_dispatch_pack_quant")


def dispatch_transfer(d: Desc, send: Sequence, plan_ws, recv: Sequence, stream=None) -> None:
    _check(_lib.ep_dispatch_transfer(ctypes.byref(d), _planes(send), _addr(plan_ws),
                                     _planes(recv), _stream(stream)), "ep_dispatch_transfer")


def dispatch_unpack(d: Desc, recv: Sequence, plan_ws, grouped: Sequence, stream=None) -> None:
    _check(_lib.ep_dispatch_unpack(ctypes.byref(d), _planes(recv), _addr(plan_ws),
                                   _planes(grouped), _stream(stream)), "ep_dispatch_unpack")


def dispatch_recv(d: Desc, send: Sequence, plan_ws, grouped: Sequence, stream=None) -> None:
    _check(_lib.ep_dispatch_recv(ctypes.byref(d), _planes(send), _addr(plan_ws),
                                 _planes(grouped), _stream(stream)), "ep_dispatch_recv")


def dispatch_send(d: Desc, topk_idx, x: Sequence, plan_ws, send: Sequence, priv: Sequence,
                  priv_rows: int, status, stream=None) -> None:
    _check(_lib.ep_dispatch_send(ctypes.byref(d), _addr(topk_idx), _planes(x), _addr(plan_ws),
                                 _planes(send), _planes(priv), int(priv_rows), _addr(status),
                                 _stream(stream)), "ep_dispatch_send")


def dispatch_recv_split(d: Desc, send: Sequence, priv: Sequence, priv_rows: int, plan_ws,
                        grouped: Sequence, status, stream=None) -> None:
    _check(_lib.ep_dispatch_recv_split(ctypes.byref(d), _planes(send), _planes(priv),
                                       int(priv_rows), _addr(plan_ws), _planes(grouped),
                                       _addr(status), _stream(stream)), "ep_dispatch_recv_split")


def dispatch_send_plan(d: Desc, topk_idx, plan_ws, status, stream=None) -> None:
    _check(_lib.ep_dispatch_send_plan(ctypes.byref(d), _addr(topk_idx), _addr(plan_ws),
                                      _addr(status), _stream(stream)), "ep_dispatch_send_plan")


def dispatch_send_pack(d: Desc, topk_idx, x: Sequence, plan_ws, send: Sequence, priv: Sequence,
                       priv_rows: int, stream=None) -> None:
    _check(_lib.ep_dispatch_send_pack(ctypes.byref(d), _addr(topk_idx), _planes(x),
                                      _addr(plan_ws), _planes(send), _planes(priv),
                                      int(priv_rows), _stream(stream)), "ep_dispatch_send_pack")


def dispatch_recv_plan(d: Desc, plan_ws, status, stream=None) -> None:
    _check(_lib.ep_dispatch_recv_plan(ctypes.byref(d), _addr(plan_ws), _addr(status),
                                      _stream(stream)), "ep_dispatch_recv_plan")


def dispatch_recv_pull(d: Desc, send: Sequence, priv: Sequence, priv_rows: int, plan_ws,
                       grouped: Sequence, stream=None) -> None:
    _check(_lib.ep_dispatch_recv_pull(ctypes.byref(d), _planes(send), _planes(priv),
                                      int(priv_rows), _addr(plan_ws), _planes(grouped),
                                      _stream(stream)), "ep_dispatch_recv_pull")


def priv_buffers(d: Desc, priv_rows: int, device="cuda") -> list:
    """Private regions of a split dispatch: per plane [N][N][P][row_p] bytes."""
    import torch
    N = d.n_ranks
    return [torch.empty((N, N, priv_rows, row_bytes(d, p)), dtype=torch.uint8, device=device)
            for p in range(num_planes(d))]


def expert_stub(d: Desc, grouped: Sequence, alpha, plan_ws, expert_out, stream=None) -> None:
    _check(_lib.ep_expert_stub(ctypes.byref(d), _planes(grouped), _addr(alpha), _addr(plan_ws),
                               _addr(expert_out), _stream(stream)), "ep_expert_stub")


def combine(d: Desc, expert_out, weights, plan_ws, out, stream=None) -> None:
    _check(_lib.ep_combine(ctypes.byref(d), _addr(expert_out), _addr(weights), _addr(plan_ws),
                           _addr(out), _stream(stream)), "ep_combine")


def combine_presum(d: Desc, expert_out, weights, plan_ws, partial, out, stream=None) -> None:
    _check(_lib.ep_combine_presum(ctypes.byref(d), _addr(expert_out), _addr(weights),
                                  _addr(plan_ws), _addr(partial), _addr(out), _stream(stream)),
           "ep_combine_presum")


class KvRegion(ctypes.Structure):
    """ep_kv_region: src_off, dst_off, bytes, first (int64 each)."""
    _fields_ = [("src_off", ctypes.c_int64), ("dst_off", ctypes.c_int64),
                ("bytes", ctypes.c_int64), ("first", ctypes.c_int64)]


def kv_plan(n_tokens: int, token_bytes: int, src_block_tokens: int, src_blocks,
            dst_block_tokens: int, dst_blocks, merge: bool = True):
    """Host-only region planner; returns an int64 numpy array [m, 4] of
    (src_off, dst_off, bytes, first)."""
    import numpy as np
    sb = np.ascontiguousarray(src_blocks, dtype=np.int32)
    db = np.ascontiguousarray(dst_blocks, dtype=np.int32)
    cap = max(int(n_tokens), 1)
    out = np.zeros((cap, 4), np.int64)
    m = _lib.ep_kv_plan(int(n_tokens), int(token_bytes), int(src_block_tokens),
                        sb.ctypes.data, int(dst_block_tokens), db.ctypes.data, int(bool(merge)),
                        out.ctypes.data, cap)
    if m < 0:
        raise EPError(int(m), "ep_kv_plan", _lib.ep_last_error().decode())
    return out[:m].copy()


def kv_push(ranks: int, regions, n_regions: int, total_bytes: int, src_pool, src_rank_bytes: int,
            dst_pool, dst_rank_bytes: int, notify, status, stream=None) -> None:
    _check(_lib.ep_kv_push(int(ranks), _addr(regions), int(n_regions), int(total_bytes),
                           _addr(src_pool), int(src_rank_bytes), _addr(dst_pool),
                           int(dst_rank_bytes), _addr(notify), _addr(status),
                           _stream(stream)), "ep_kv_push")


def kv_push_staged(ranks: int, regions, n_regions: int, total_bytes: int, src_pool,
                   src_rank_bytes: int, dst_pool, dst_rank_bytes: int, bounce, bounce_slots: int,
                   notify, status, stream=None) -> None:
    _check(_lib.ep_kv_push_staged(int(ranks), _addr(regions), int(n_regions), int(total_bytes),
                                  _addr(src_pool), int(src_rank_bytes), _addr(dst_pool),
                                  int(dst_rank_bytes), _addr(bounce), int(bounce_slots),
                                  _addr(notify), _addr(status), _stream(stream)),
           "ep_kv_push_staged")


def kv_push_staged_static(ranks: int, regions, n_regions: int, total_bytes: int, src_pool,
                          src_rank_bytes: int, dst_pool, dst_rank_bytes: int, bounce_slots: int,
                          notify, status, stream=None) -> None:
    _check(_lib.ep_kv_push_staged_static(int(ranks), _addr(regions), int(n_regions),
                                         int(total_bytes), _addr(src_pool), int(src_rank_bytes),
                                         _addr(dst_pool), int(dst_rank_bytes), int(bounce_slots),
                                         _addr(notify), _addr(status), _stream(stream)),
           "ep_kv_push_staged_static")


def probe_copy(dst, src, nbytes: int, stream=None) -> None:
    _check(_lib.ep_probe_copy(_addr(dst), _addr(src), nbytes, _stream(stream)), "ep_probe_copy")


def probe_pattern(dst, src, table, rows: int, indexed_rows: int, row_bytes: int,
                  piece_bytes: int, fan_in: int = 1, in_flight: int = 0,
                  mode: int = EP_PROBE_COPY, flags: int = 0, waves: int = 0,
                  stream=None) -> None:
    """in_flight 0 means all fan_in rows at once (1 for a scatter)."""
    if not in_flight:
        in_flight = 1 if mode in (EP_PROBE_SCATTER, EP_PROBE_SCATTER_WIDE) else fan_in
    _check(_lib.ep_probe_pattern(_addr(dst), _addr(src), _addr(table), int(rows),
                                 int(indexed_rows), int(row_bytes), int(piece_bytes),
                                 int(fan_in), int(in_flight), int(mode), int(flags), int(waves),
                                 _stream(stream)), "ep_probe_pattern")


# ---------------------------------------------------------------------------
# Device buffers for one descriptor (torch allocations; plumbing only)
# ---------------------------------------------------------------------------

class Buffers:
    """Caller-owned device buffers of one dispatch/combine step."""

    def __init__(self, d: Desc, device="cuda", staged: bool = False):
        import torch
        self.desc = d
        N, T, H, R = d.n_ranks, d.tokens, d.hidden, d.topk
        cap = capacity(d)
        if cap < 0:
            raise EPError(EP_ERR_INVALID_ARG, "Buffers", last_error())
        self.cap = cap
        self.planes = num_planes(d)
        rows = [row_bytes(d, p) for p in range(self.planes)]
        u8 = torch.uint8
        self.idx = torch.empty((N, T, R), dtype=torch.int32, device=device)
        self.weights = torch.empty((N, T, R), dtype=torch.float32, device=device)
        self.x = [torch.empty((N, T, r), dtype=u8, device=device) for r in rows]
        self.send = [torch.empty((N, T * R, r), dtype=u8, device=device) for r in rows]
        self.grouped = [torch.empty((N, cap, r), dtype=u8, device=device) for r in rows]
        self.recv = ([torch.empty((N, cap, r), dtype=u8, device=device) for r in rows]
                     if staged else None)
        self.expert_out = torch.empty((N, cap, H), dtype=torch.int16, device=device)
        self.out = torch.empty((N, T, H), dtype=torch.int16, device=device)
        self.plan_ws = torch.empty(plan_bytes(d), dtype=u8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
