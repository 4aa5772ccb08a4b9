"""ctypes front end of the double-precision CPU oracle (pic_oracle.c).

TEST INFRASTRUCTURE ONLY: the product package never imports this module.  The
test suite, the smoke check and the benchmark's CPU-baseline leg use it.

Every function takes a workload object by duck typing: any object carrying the
arrays described in pic_oracle.c's header (pool_k, pool_v, block_table,
kv_len, kv_pos, q, q_start, q_pos) and the head geometry (num_q_heads,
num_kv_heads, head_dim, rope_theta).  Arrays are read, never written, except by
`fuse`, which works on copies and returns them.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pic_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i32p = C.POINTER(C.c_int32)
_u16p = C.POINTER(C.c_uint16)
_f64p = C.POINTER(C.c_double)


class _Problem(C.Structure):
    _fields_ = [
        ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("batch", C.c_int32), ("num_blocks", C.c_int32), ("max_blocks", C.c_int32),
        ("rope_theta", C.c_double),
        ("pool_k", _u16p), ("pool_v", _u16p),
        ("block_table", _i32p), ("kv_len", _i32p), ("kv_pos", _i32p),
        ("q", _u16p), ("q_start", _i32p), ("q_pos", _i32p),
    ]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE double arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        h = C.CDLL(build())
        h.oracle_rope.argtypes = [C.c_int32, C.c_double, C.c_int32, _f64p, _f64p]
        h.oracle_rope.restype = None
        h.oracle_attention.argtypes = [C.POINTER(_Problem), C.c_int32, _i32p, _i32p, _f64p, _f64p]
        h.oracle_attention.restype = C.c_int
        h.oracle_mass.argtypes = [C.POINTER(_Problem), C.c_int32, _f64p]
        h.oracle_mass.restype = C.c_int
        h.oracle_key_norm.argtypes = [C.POINTER(_Problem), C.c_int32, _f64p]
        h.oracle_key_norm.restype = C.c_int
        h.oracle_select.argtypes = [C.c_int32, _i32p, _i32p, _i32p, C.c_double, _f64p, C.c_int32,
                                    _i32p, _i32p, _i32p, _i32p, C.c_int32]
        h.oracle_select.restype = C.c_int32
        h.oracle_fuse.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _i32p,
                                  _i32p, _i32p, _u16p, _u16p, _i32p, _i32p, _u16p, _u16p]
        h.oracle_fuse.restype = C.c_int
        _lib = h
    return _lib


def _ptr(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


def _problem(w, keep: list) -> _Problem:
    arrs = dict(
        pool_k=np.ascontiguousarray(w.pool_k, np.uint16), pool_v=np.ascontiguousarray(w.pool_v, np.uint16),
        block_table=np.ascontiguousarray(w.block_table, np.int32),
        kv_len=np.ascontiguousarray(w.kv_len, np.int32), kv_pos=np.ascontiguousarray(w.kv_pos, np.int32),
        q=np.ascontiguousarray(w.q, np.uint16), q_start=np.ascontiguousarray(w.q_start, np.int32),
        q_pos=np.ascontiguousarray(w.q_pos, np.int32))
    keep.append(arrs)
    return _Problem(
        int(w.num_q_heads), int(w.num_kv_heads), int(w.head_dim), int(arrs["kv_len"].shape[0]),
        int(arrs["pool_k"].shape[0]), int(arrs["block_table"].shape[1]), float(w.rope_theta),
        _ptr(arrs["pool_k"], _u16p), _ptr(arrs["pool_v"], _u16p), _ptr(arrs["block_table"], _i32p),
        _ptr(arrs["kv_len"], _i32p), _ptr(arrs["kv_pos"], _i32p), _ptr(arrs["q"], _u16p),
        _ptr(arrs["q_start"], _i32p), _ptr(arrs["q_pos"], _i32p))


def rope(d: int, theta: float, pos: int, x: np.ndarray) -> np.ndarray:
    """The oracle's rotation of one vector to logical position `pos`."""
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty_like(x)
    lib().oracle_rope(int(d), float(theta), int(pos), _ptr(x, _f64p), _ptr(y, _f64p))
    return y


def attention(w, rows: Optional[Tuple[np.ndarray, np.ndarray]] = None):
    """(out, lse) in float64.  rows=None: every (t, h), out [total_q, Hq, d],
    lse [total_q, Hq].  rows=(t, h) arrays: out [n, d], lse [n]."""
    keep: list = []
    p = _problem(w, keep)
    d = int(w.head_dim)
    if rows is None:
        nt = int(np.asarray(w.q).shape[0])
        out = np.zeros((nt, int(w.num_q_heads), d), np.float64)
        lse = np.zeros((nt, int(w.num_q_heads)), np.float64)
        rc = lib().oracle_attention(C.byref(p), -1, None, None, _ptr(out, _f64p), _ptr(lse, _f64p))
    else:
        t = np.ascontiguousarray(rows[0], np.int32)
        h = np.ascontiguousarray(rows[1], np.int32)
        out = np.zeros((t.shape[0], d), np.float64)
        lse = np.zeros(t.shape[0], np.float64)
        rc = lib().oracle_attention(C.byref(p), int(t.shape[0]), _ptr(t, _i32p), _ptr(h, _i32p),
                                    _ptr(out, _f64p), _ptr(lse, _f64p))
    if rc != 0:
        raise ValueError("oracle_attention: bad row list")
    return out, lse


def mass(w) -> np.ndarray:
    """Selection mass [B, max_blocks*16] in float64 (zero beyond kv_len)."""
    keep: list = []
    p = _problem(w, keep)
    stride = int(np.asarray(w.kv_pos).shape[1])
    m = np.zeros((int(np.asarray(w.kv_len).shape[0]), stride), np.float64)
    lib().oracle_mass(C.byref(p), stride, _ptr(m, _f64p))
    return m


def key_norm(w) -> np.ndarray:
    """Anchor score [B, max_blocks*16] in float64: squared norm of each usable
    slot's stored key over all kv heads (zero beyond kv_len and for unusable
    slots)."""
    keep: list = []
    p = _problem(w, keep)
    stride = int(np.asarray(w.kv_pos).shape[1])
    m = np.zeros((int(np.asarray(w.kv_len).shape[0]), stride), np.float64)
    lib().oracle_key_norm(C.byref(p), stride, _ptr(m, _f64p))
    return m


def select(w, mass_arr: np.ndarray, ratio: Optional[float] = None):
    """Per-span top fraction of the score mass_arr (selection mass or anchor
    key norm): (sel_off [n_spans+1], sel_idx [total])."""
    ratio = float(w.ratio if ratio is None else ratio)
    sr = np.ascontiguousarray(w.span_req, np.int32)
    ss = np.ascontiguousarray(w.span_start, np.int32)
    sl = np.ascontiguousarray(w.span_len, np.int32)
    kv_pos = np.ascontiguousarray(w.kv_pos, np.int32)
    kv_len = np.ascontiguousarray(w.kv_len, np.int32)
    m = np.ascontiguousarray(mass_arr, np.float64)
    n = int(sr.shape[0])
    cap = int(sl.sum()) + 1
    off = np.zeros(n + 1, np.int32)
    idx = np.zeros(cap, np.int32)
    tot = lib().oracle_select(n, _ptr(sr, _i32p), _ptr(ss, _i32p), _ptr(sl, _i32p), ratio,
                              _ptr(m, _f64p), int(kv_pos.shape[1]), _ptr(kv_pos, _i32p),
                              _ptr(kv_len, _i32p), _ptr(off, _i32p), _ptr(idx, _i32p), cap)
    if tot < 0:
        raise ValueError("oracle_select: capacity")
    return off, idx[:tot].copy()


def fuse(w, sel_idx: np.ndarray, sel_req_off: np.ndarray, fresh_k: np.ndarray, fresh_v: np.ndarray):
    """Fused copies: (pool_k, pool_v, kv_pos, kv_len)."""
    pool_k = np.ascontiguousarray(w.pool_k, np.uint16).copy()
    pool_v = np.ascontiguousarray(w.pool_v, np.uint16).copy()
    kv_pos = np.ascontiguousarray(w.kv_pos, np.int32).copy()
    kv_len = np.ascontiguousarray(w.kv_len, np.int32).copy()
    bt = np.ascontiguousarray(w.block_table, np.int32)
    si = np.ascontiguousarray(sel_idx, np.int32)
    so = np.ascontiguousarray(sel_req_off, np.int32)
    fk = np.ascontiguousarray(fresh_k, np.uint16)
    fv = np.ascontiguousarray(fresh_v, np.uint16)
    if si.size == 0:
        si = np.zeros(1, np.int32)
    if fk.size == 0:
        fk = np.zeros(1, np.uint16)
        fv = np.zeros(1, np.uint16)
    rc = lib().oracle_fuse(int(kv_len.shape[0]), int(w.num_kv_heads), int(w.head_dim),
                           int(pool_k.shape[0]), int(bt.shape[1]), _ptr(bt, _i32p),
                           _ptr(kv_len, _i32p), _ptr(kv_pos, _i32p), _ptr(pool_k, _u16p),
                           _ptr(pool_v, _u16p), _ptr(si, _i32p), _ptr(so, _i32p),
                           _ptr(fk, _u16p), _ptr(fv, _u16p))
    if rc != 0:
        raise ValueError("oracle_fuse: a fused slot has no private block")
    return pool_k, pool_v, kv_pos, kv_len
