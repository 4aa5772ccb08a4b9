"""ctypes binding of libpicattn.so (include/pic_attn.h), same entry-point names.

Argument marshalling only: torch tensors supply device memory and
torch.cuda streams supply the hipStream_t; every step of the computation runs
in the library's HIP kernels.  Loading fails loudly when the library is
missing: there is no fallback path.

bf16 data travels as torch.int16 tensors holding bf16 bit patterns (the
library's uint16_t).
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpicattn.so")

PIC_OK, PIC_ERR_INVALID_ARG, PIC_ERR_UNSUPPORTED, PIC_ERR_WORKSPACE, PIC_ERR_HIP = range(5)
PIC_OP_PREFILL, PIC_OP_DECODE, PIC_OP_SELECT, PIC_OP_ANCHOR = range(4)
PIC_BLOCK_SIZE = 16

_vp = C.c_void_p
_i32 = C.c_int32


class PicConfig(C.Structure):
    _fields_ = [("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("block_size", _i32), ("max_position", _i32), ("rope_theta", C.c_double),
                ("keys_prerotated", _i32)]


class PicKvPool(C.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("num_blocks", _i32)]


class PicReqTable(C.Structure):
    _fields_ = [("batch", _i32), ("max_blocks", _i32), ("max_kv_len", _i32),
                ("block_table", _vp), ("kv_len", _vp), ("kv_pos", _vp)]


class PicQueries(C.Structure):
    _fields_ = [("q", _vp), ("q_start", _vp), ("q_pos", _vp), ("total_q", _i32), ("max_q_len", _i32)]


class PicSpans(C.Structure):
    _fields_ = [("n_spans", _i32), ("span_req", _vp), ("span_start", _vp), ("span_len", _vp),
                ("sel_off", _vp)]


class PicError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """Load libpicattn.so (built by __graft_entry__.build() or build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m position_independent_attention_amd.build`")
        h = C.CDLL(LIB_PATH)
        P = C.POINTER
        h.pic_ctx_create.argtypes = [P(PicConfig), P(_vp)]
        h.pic_ctx_create.restype = C.c_int
        h.pic_ctx_destroy.argtypes = [_vp]
        h.pic_ctx_destroy.restype = None
        h.pic_status_str.argtypes = [C.c_int]
        h.pic_status_str.restype = C.c_char_p
        h.pic_ctx_last_error.argtypes = [_vp]
        h.pic_ctx_last_error.restype = C.c_char_p
        h.pic_workspace_bytes.argtypes = [_vp, C.c_int, P(PicReqTable), _i32, _i32, P(C.c_size_t)]
        h.pic_workspace_bytes.restype = C.c_int
        h.pic_select_offsets.argtypes = [_i32, _vp, C.c_double, _vp]
        h.pic_select_offsets.restype = C.c_int
        h.pic_attn_prefill.argtypes = [_vp, P(PicKvPool), P(PicReqTable), P(PicQueries), _vp, _vp, _vp,
                                       C.c_size_t, _vp]
        h.pic_attn_prefill.restype = C.c_int
        h.pic_attn_decode.argtypes = [_vp, P(PicKvPool), P(PicReqTable), _vp, _vp, _vp, _vp, _vp,
                                      C.c_size_t, _vp]
        h.pic_attn_decode.restype = C.c_int
        h.qc_score_select.argtypes = [_vp, P(PicKvPool), P(PicReqTable), P(PicQueries), _vp, P(PicSpans),
                                      _i32, _vp, _vp, _vp, C.c_size_t, _vp]
        h.qc_score_select.restype = C.c_int
        h.qc_score_select_noalloc.argtypes = [_vp, P(PicKvPool), P(PicReqTable), P(PicQueries), _vp,
                                              P(PicSpans), _i32, _vp, _vp, _vp]
        h.qc_score_select_noalloc.restype = C.c_int
        h.qc_anchor_select.argtypes = [_vp, P(PicKvPool), P(PicReqTable), P(PicSpans), _i32, _vp, _vp, _vp,
                                       C.c_size_t, _vp]
        h.qc_anchor_select.restype = C.c_int
        h.pic_block_cache_create.argtypes = [_i32, P(_vp)]
        h.pic_block_cache_create.restype = C.c_int
        h.pic_block_cache_destroy.argtypes = [_vp]
        h.pic_block_cache_destroy.restype = None
        h.pic_block_map.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, P(_i32)]
        h.pic_block_map.restype = C.c_int
        h.kv_fuse_scatter.argtypes = [_vp, P(PicKvPool), P(PicReqTable), _vp, _vp, _vp, _vp, _i32, _i32, _vp]
        h.kv_fuse_scatter.restype = C.c_int
        h.pic_timing_start.argtypes = [_vp, _i32]
        h.pic_timing_start.restype = C.c_int
        h.pic_timing_stop.argtypes = [_vp, _vp, _vp, _i32, P(_i32)]
        h.pic_timing_stop.restype = C.c_int
        _lib = h
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


class Context:
    """pic_ctx_create / pic_ctx_destroy.  Create it with the target device current."""

    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, rope_theta: float,
                 max_position: int = 65536, block_size: int = PIC_BLOCK_SIZE, keys_prerotated: bool = False):
        self.cfg = PicConfig(num_q_heads, num_kv_heads, head_dim, block_size, max_position, rope_theta,
                             1 if keys_prerotated else 0)
        h = _vp()
        st = lib().pic_ctx_create(C.byref(self.cfg), C.byref(h))
        if st != PIC_OK:
            raise PicError(st, "pic_ctx_create")
        self.handle = h

    def last_error(self) -> str:
        return lib().pic_ctx_last_error(self.handle).decode()

    def close(self):
        if getattr(self, "handle", None):
            lib().pic_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _check(ctx: Context, st: int, what: str):
    if st != PIC_OK:
        raise PicError(st, f"{what}: {lib().pic_status_str(st).decode()} ({ctx.last_error()})")


@dataclasses.dataclass
class DeviceCache:
    """Device copies of a pool + request table (+ queries and spans)."""
    pool_k: object
    pool_v: object
    block_table: object
    kv_len: object
    kv_pos: object
    max_kv_len: int
    q: object = None
    q_start: object = None
    q_pos: object = None
    total_q: int = 0
    max_q_len: int = 0
    span_req: object = None
    span_start: object = None
    span_len: object = None
    sel_off: object = None
    n_spans: int = 0

    def pool(self) -> PicKvPool:
        return PicKvPool(_ptr(self.pool_k), _ptr(self.pool_v), int(self.pool_k.shape[0]))

    def req(self) -> PicReqTable:
        return PicReqTable(int(self.block_table.shape[0]), int(self.block_table.shape[1]),
                           int(self.max_kv_len), _ptr(self.block_table), _ptr(self.kv_len), _ptr(self.kv_pos))

    def queries(self) -> PicQueries:
        return PicQueries(_ptr(self.q), _ptr(self.q_start), _ptr(self.q_pos), int(self.total_q),
                          int(self.max_q_len))

    def spans(self) -> PicSpans:
        return PicSpans(int(self.n_spans), _ptr(self.span_req), _ptr(self.span_start), _ptr(self.span_len),
                        _ptr(self.sel_off))


def to_device(w, device="cuda", sel_off: Optional[np.ndarray] = None, max_kv_len: Optional[int] = None
              ) -> DeviceCache:
    """Upload a host workload (see workloads.Workload) with torch as the allocator."""
    import torch

    def t(a, dt=None):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(device)

    dc = DeviceCache(pool_k=t(w.pool_k), pool_v=t(w.pool_v), block_table=t(w.block_table),
                     kv_len=t(w.kv_len), kv_pos=t(w.kv_pos),
                     max_kv_len=int(max_kv_len if max_kv_len is not None else w.max_kv_len),
                     q=t(w.q), q_start=t(w.q_start), q_pos=t(w.q_pos), total_q=int(w.total_q),
                     max_q_len=int(w.max_q_len))
    if len(w.span_req):
        dc.span_req, dc.span_start, dc.span_len = t(w.span_req), t(w.span_start), t(w.span_len)
        dc.n_spans = int(len(w.span_req))
        if sel_off is not None:
            dc.sel_off = t(np.asarray(sel_off, np.int32))
    return dc


# ------------------------------------------------------------ entry points

def pic_workspace_bytes(ctx: Context, op: int, req: PicReqTable, total_q: int, max_q_len: int) -> int:
    n = C.c_size_t(0)
    _check(ctx, lib().pic_workspace_bytes(ctx.handle, op, C.byref(req), total_q, max_q_len, C.byref(n)),
           "pic_workspace_bytes")
    return int(n.value)


def pic_timing_start(ctx: Context, capacity: int):
    _check(ctx, lib().pic_timing_start(ctx.handle, int(capacity)), "pic_timing_start")


def pic_timing_stop(ctx: Context, cap: int):
    """-> (ms, ops): the recorded kernel intervals in call order."""
    ms = np.zeros(max(1, cap), np.float32)
    ops = np.zeros(max(1, cap), np.int32)
    n = _i32(0)
    _check(ctx, lib().pic_timing_stop(ctx.handle, ms.ctypes.data, ops.ctypes.data, int(cap), C.byref(n)),
           "pic_timing_stop")
    k = min(int(n.value), cap)
    return ms[:k].copy(), ops[:k].copy()


def pic_select_offsets(span_len: np.ndarray, ratio: float) -> np.ndarray:
    sl = np.ascontiguousarray(span_len, np.int32)
    off = np.zeros(len(sl) + 1, np.int32)
    st = lib().pic_select_offsets(len(sl), sl.ctypes.data if len(sl) else None, float(ratio), off.ctypes.data)
    if st != PIC_OK:
        raise PicError(st, "pic_select_offsets")
    return off


def _workspace(ctx, op, req, total_q, max_q_len, ws, device):
    import torch
    need = pic_workspace_bytes(ctx, op, req, total_q, max_q_len)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return ws, need


def pic_attn_prefill(ctx: Context, dc: DeviceCache, out, lse=None, ws=None, stream=None):
    pool, req, qs = dc.pool(), dc.req(), dc.queries()
    ws, _ = _workspace(ctx, PIC_OP_PREFILL, req, qs.total_q, qs.max_q_len, ws, dc.pool_k.device)
    st = lib().pic_attn_prefill(ctx.handle, C.byref(pool), C.byref(req), C.byref(qs), _ptr(out), _ptr(lse),
                                _ptr(ws), ws.numel(), _stream(stream))
    _check(ctx, st, "pic_attn_prefill")
    return out, lse


def pic_attn_decode(ctx: Context, dc: DeviceCache, q, q_pos, out, lse=None, ws=None, stream=None):
    pool, req = dc.pool(), dc.req()
    ws, _ = _workspace(ctx, PIC_OP_DECODE, req, 0, 0, ws, dc.pool_k.device)
    st = lib().pic_attn_decode(ctx.handle, C.byref(pool), C.byref(req), _ptr(q), _ptr(q_pos), _ptr(out),
                               _ptr(lse), _ptr(ws), ws.numel(), _stream(stream))
    _check(ctx, st, "pic_attn_decode")
    return out, lse


def qc_score_select(ctx: Context, dc: DeviceCache, lse, max_sel: int, sel_idx, mass=None, ws=None,
                    stream=None):
    pool, req, qs, sp = dc.pool(), dc.req(), dc.queries(), dc.spans()
    ws, _ = _workspace(ctx, PIC_OP_SELECT, req, qs.total_q, qs.max_q_len, ws, dc.pool_k.device)
    st = lib().qc_score_select(ctx.handle, C.byref(pool), C.byref(req), C.byref(qs), _ptr(lse), C.byref(sp),
                               int(max_sel), _ptr(sel_idx), _ptr(mass), _ptr(ws), ws.numel(), _stream(stream))
    _check(ctx, st, "qc_score_select")
    return sel_idx, mass


def qc_score_select_noalloc(ctx: Context, dc: DeviceCache, lse, max_sel: int, sel_idx, mass=None, stream=None):
    """qc_score_select with the library's per-GPU scratch as its workspace
    (no device allocation)."""
    pool, req, qs, sp = dc.pool(), dc.req(), dc.queries(), dc.spans()
    st = lib().qc_score_select_noalloc(ctx.handle, C.byref(pool), C.byref(req), C.byref(qs), _ptr(lse),
                                       C.byref(sp), int(max_sel), _ptr(sel_idx), _ptr(mass), _stream(stream))
    _check(ctx, st, "qc_score_select_noalloc")
    return sel_idx, mass


def qc_anchor_select(ctx: Context, dc: DeviceCache, max_sel: int, sel_idx, norm=None, ws=None, stream=None):
    """Per-span anchors by stored-key norm (dc.sel_off holds the per-span budget
    CSR, e.g. from pic_select_offsets with the anchor fraction)."""
    pool, req, sp = dc.pool(), dc.req(), dc.spans()
    ws, _ = _workspace(ctx, PIC_OP_ANCHOR, req, 0, 0, ws, dc.pool_k.device)
    st = lib().qc_anchor_select(ctx.handle, C.byref(pool), C.byref(req), C.byref(sp), int(max_sel), _ptr(sel_idx),
                                _ptr(norm), _ptr(ws), ws.numel(), _stream(stream))
    _check(ctx, st, "qc_anchor_select")
    return sel_idx, norm


def kv_fuse_scatter(ctx: Context, dc: DeviceCache, sel_idx, sel_req_off, k_new, v_new, n_sel: int,
                    max_rows_per_req: int, stream=None):
    pool, req = dc.pool(), dc.req()
    st = lib().kv_fuse_scatter(ctx.handle, C.byref(pool), C.byref(req), _ptr(sel_idx), _ptr(sel_req_off),
                               _ptr(k_new), _ptr(v_new), int(n_sel), int(max_rows_per_req), _stream(stream))
    _check(ctx, st, "kv_fuse_scatter")


class BlockCache:
    """pic_block_cache_*: span reuse by block hashing (host only)."""

    def __init__(self, num_blocks: int):
        h = _vp()
        st = lib().pic_block_cache_create(int(num_blocks), C.byref(h))
        if st != PIC_OK:
            raise PicError(st, "pic_block_cache_create")
        self.handle = h

    def map_request(self, tokens, pad_token: int, ssep_token: int, pdep_token: int):
        """(block_table, kv_pos[:n_tokens], miss) as numpy int32 arrays."""
        import numpy as np
        t = np.ascontiguousarray(tokens, np.int32)
        nb = (t.shape[0] + PIC_BLOCK_SIZE - 1) // PIC_BLOCK_SIZE
        table = np.zeros(max(nb, 1), np.int32)
        miss = np.zeros(max(nb, 1), np.int32)
        pos = np.zeros(max(nb, 1) * PIC_BLOCK_SIZE, np.int32)
        n = _i32()
        st = lib().pic_block_map(self.handle, t.ctypes.data_as(_vp), int(t.shape[0]), int(pad_token),
                                 int(ssep_token), int(pdep_token), table.ctypes.data_as(_vp), int(nb),
                                 pos.ctypes.data_as(_vp), miss.ctypes.data_as(_vp), C.byref(n))
        if st != PIC_OK:
            raise PicError(st, "pic_block_map")
        return table[:n.value], pos[:t.shape[0]], miss[:n.value]

    def close(self):
        if self.handle:
            lib().pic_block_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
