"""Float64 CPU oracle for the CSA/HCA hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and it imports nothing from them.

The arithmetic lives in ``lca_oracle.c`` (plain C, float64, fixed
left-to-right loops, built without fast-math and without FMA contraction).
This module only marshals numpy arrays into it.  See ``lca_oracle.c`` for the
passages each function follows and the readings taken where the pages are
silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lca_oracle.c")
LIB = os.path.join(HERE, "liblca_oracle.so")

F32, BF16, FP8E4M3, MXFP4 = 0, 1, 2, 3

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (float64, no fast-math, no FP contraction)."""
    if force or not os.path.exists(LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", LIB + ".tmp", SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.orc_e4m3_value.restype = dbl
        L.orc_e4m3_value.argtypes = [i32]
        L.orc_e2m1_value.restype = dbl
        L.orc_e2m1_value.argtypes = [i32]
        L.orc_e4m3_encode.restype = i32
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e2m1_encode.restype = i32
        L.orc_e2m1_encode.argtypes = [dbl]
        L.orc_bf16_value.restype = dbl
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_encode.restype = ctypes.c_uint16
        L.orc_bf16_encode.argtypes = [ctypes.c_float]
        L.orc_decode.restype = None
        L.orc_decode.argtypes = [vp, i32, vp, i64, vp]
        L.orc_encode.restype = None
        L.orc_encode.argtypes = [vp, i64, i32, vp, vp]
        L.orc_pool.restype = None
        L.orc_pool.argtypes = [vp, vp, vp, i64, i32, i32, vp]
        L.orc_pool_variant.restype = None
        L.orc_pool_variant.argtypes = [vp, vp, i32, vp, i64, i32, i32, i32, vp]
        L.orc_index_score.restype = dbl
        L.orc_index_score.argtypes = [vp, vp, vp, i32, i32]
        L.orc_select_topk.restype = None
        L.orc_select_topk.argtypes = [vp, i64, i32, vp, vp]
        L.orc_index_topk.restype = None
        L.orc_index_topk.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i64, i32,
                                     vp, vp, vp]
        L.orc_attend_row.restype = None
        L.orc_attend_row.argtypes = [vp, vp, i64, vp, i64, vp, dbl, i32, i32, vp, vp]
        L.orc_attend.restype = None
        L.orc_attend.argtypes = [vp, vp, i32, vp, i64, vp, i32, vp, vp, i32, i64, vp, vp, vp,
                                 dbl, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_num_threads.restype = i32
        L.orc_num_threads.argtypes = []
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# codecs
# --------------------------------------------------------------------------
def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(float(y))


def e2m1_encode(y: float) -> int:
    return lib().orc_e2m1_encode(float(y))


def encode(v, dt):
    """Encode fp32 values (last dim a multiple of 64) to a storage type.

    Returns (codes, scales): FP8 -> uint8 same shape + float32 [..., D/64];
    MXFP4 -> uint8 [..., D/2] + uint8 E8M0 [..., D/32]; BF16 -> uint16, None;
    F32 -> float32, None."""
    v = _c(v, np.float32)
    shape = v.shape
    n = v.size
    D = shape[-1]
    if dt == F32:
        return v.copy(), None
    if dt == BF16:
        out = np.empty(shape, np.uint16)
        lib().orc_encode(_p(v), n, dt, _p(out), None)
        return out, None
    if dt == FP8E4M3:
        assert D % 64 == 0
        out = np.empty(shape, np.uint8)
        sc = np.empty(shape[:-1] + (D // 64,), np.float32)
        lib().orc_encode(_p(v), n, dt, _p(out), _p(sc))
        return out, sc
    if dt == MXFP4:
        assert D % 32 == 0
        out = np.empty(shape[:-1] + (D // 2,), np.uint8)
        sc = np.empty(shape[:-1] + (D // 32,), np.uint8)
        lib().orc_encode(_p(v), n, dt, _p(out), _p(sc))
        return out, sc
    raise ValueError(dt)


def decode(codes, dt, scales=None, D=None):
    """Decode storage to float64; D is the logical last dim (needed for MXFP4)."""
    if dt == F32:
        c = _c(codes, np.float32)
        shape = c.shape
    elif dt == BF16:
        c = _c(codes, np.uint16)
        shape = c.shape
    elif dt == FP8E4M3:
        c = _c(codes, np.uint8)
        shape = c.shape
        scales = _c(scales, np.float32)
    elif dt == MXFP4:
        c = _c(codes, np.uint8)
        shape = c.shape[:-1] + (c.shape[-1] * 2,)
        scales = _c(scales, np.uint8)
    else:
        raise ValueError(dt)
    n = int(np.prod(shape))
    out = np.empty(shape, np.float64)
    lib().orc_decode(_p(c), dt, _p(scales), n, _p(out))
    return out


# --------------------------------------------------------------------------
# O1 pooling
# --------------------------------------------------------------------------
def pool(x, gate, bias, m):
    """Pool one sequence: x [T, D] float64, gate [T], bias [m] -> [T//m, D]."""
    x = _c(x, np.float64)
    gate = _c(gate, np.float64)
    bias = _c(bias, np.float64)
    T, D = x.shape
    nblk = T // m
    out = np.empty((nblk, D), np.float64)
    if nblk:
        lib().orc_pool(_p(x), _p(gate), _p(bias), nblk, int(m), int(D), _p(out))
    return out


def pool_variant(x, gate, bias, m, overlap=0):
    """Pooling variants (see orc_pool_variant): x [T, D]; gate [T] (one logit per
    token) or [T, D] (per channel); bias [m + overlap] or [m + overlap, D]
    matching the gate; block j pools positions j*m - overlap .. j*m + m - 1 that
    exist.  Returns [T // m, D] float64."""
    x = _c(x, np.float64)
    gate = _c(gate, np.float64)
    bias = _c(bias, np.float64)
    T, D = x.shape
    pc = 1 if gate.ndim == 2 else 0
    assert gate.shape == ((T, D) if pc else (T,))
    assert bias.shape == ((m + overlap, D) if pc else (m + overlap,))
    assert 0 <= overlap <= m
    nblk = T // m
    out = np.empty((nblk, D), np.float64)
    if nblk:
        lib().orc_pool_variant(_p(x), _p(gate), pc, _p(bias), nblk, int(m), int(overlap), int(D), _p(out))
    return out


# --------------------------------------------------------------------------
# O3/O4 indexer + top-k
# --------------------------------------------------------------------------
def index_score(q, w, kj):
    q = _c(q, np.float64)
    w = _c(w, np.float64)
    kj = _c(kj, np.float64)
    H, d = q.shape
    return lib().orc_index_score(_p(q), _p(w), _p(kj), H, d)


def select_topk(s, k):
    s = _c(s, np.float64)
    idx = np.empty(k, np.int32)
    sc = np.empty(k, np.float64)
    lib().orc_select_topk(_p(s), s.size, int(k), _p(idx), _p(sc))
    return idx, sc


def index_topk(qi, w, keys, key_dt, key_scale, n_elig, k, want_scores=False):
    """qi: float64 [B, Tq, H, d] (already decoded); w: f32 [B, Tq, H];
    keys: storage [B, N_cap, ...]; n_elig: int32 [B, Tq].
    Returns idx [B,Tq,k] int32, selected scores [B,Tq,k] float64 (0 for -1),
    and optionally all scores [B,Tq,N_cap] (eligible part valid)."""
    qi = _c(qi, np.float64)
    B, Tq, H, d = qi.shape
    assert H <= 64
    w = _c(w, np.float32)
    n_elig = _c(n_elig, np.int32)
    N_cap = keys.shape[1]
    if key_dt == F32:
        keys = _c(keys, np.float32)
    elif key_dt == BF16:
        keys = _c(keys, np.uint16)
    elif key_dt == FP8E4M3:
        keys = _c(keys, np.uint8)
        key_scale = _c(key_scale, np.float32)
    else:
        keys = _c(keys, np.uint8)
        key_scale = _c(key_scale, np.uint8)
    idx = np.empty((B, Tq, k), np.int32)
    sc = np.empty((B, Tq, k), np.float64)
    allsc = np.zeros((B, Tq, N_cap), np.float64) if want_scores else None
    lib().orc_index_topk(_p(qi), _p(w), _p(keys), key_dt, _p(key_scale), _p(n_elig), B, Tq, H,
                         d, N_cap, int(k), _p(idx), _p(sc), _p(allsc))
    if want_scores:
        return idx, sc, allsc
    return idx, sc


# --------------------------------------------------------------------------
# O5 attention
# --------------------------------------------------------------------------
def attend_row(q, ent, win, sink, tau):
    q = _c(q, np.float64)
    Hq, D = q.shape
    ent = _c(ent, np.float64).reshape(-1, D)
    win = _c(win, np.float64).reshape(-1, D)
    sink = _c(sink, np.float32)
    o = np.empty((Hq, D), np.float64)
    lse = np.empty(Hq, np.float64)
    lib().orc_attend_row(_p(q), _p(ent), ent.shape[0], _p(win), win.shape[0], _p(sink),
                         float(tau), Hq, D, _p(o), _p(lse))
    return o, lse


def attend(q, kv, kv_dt, kv_scale, sel, n_elig, win, win_dt, win_begin, win_len, sink, tau, v=None,
           v_scale=None, win_v=None):
    """q: float64 [B,Tq,Hq,D]; kv storage [B,N_cap,D] (+ fp32 scales per 64);
    sel int32 [B,Tq,k] for sparse attention or None for dense over n_elig;
    win storage [B,W_buf,D]; win_begin/win_len int32 [B,Tq]; sink f32 [Hq].
    v / v_scale / win_v: separate values in the layouts of kv / kv_scale / win
    (None: one vector per item is key and value; both v and win_v or neither).
    Returns o float64 [B,Tq,Hq,D], lse float64 [B,Tq,Hq]."""
    assert (v is None) == (win_v is None)
    q = _c(q, np.float64)
    B, Tq, Hq, D = q.shape
    N_cap = kv.shape[1]

    def store(a, sc):
        if kv_dt == F32:
            return _c(a, np.float32), None
        if kv_dt == BF16:
            return _c(a, np.uint16), None
        return _c(a, np.uint8), _c(sc, np.float32)
    kv, kv_scale = store(kv, kv_scale)
    if v is not None:
        assert v.shape == kv.shape
        v, v_scale = store(v, v_scale)
        win_v = _c(win_v, np.float32 if win_dt == F32 else np.uint16)
        assert win_v.shape == win.shape
    win = _c(win, np.float32 if win_dt == F32 else np.uint16)
    W_buf = win.shape[1]
    k = 0
    if sel is not None:
        sel = _c(sel, np.int32)
        k = sel.shape[-1]
    if n_elig is not None:
        n_elig = _c(n_elig, np.int32)
    win_begin = _c(win_begin, np.int32)
    win_len = _c(win_len, np.int32)
    sink = _c(sink, np.float32)
    o = np.empty((B, Tq, Hq, D), np.float64)
    lse = np.empty((B, Tq, Hq), np.float64)
    lib().orc_attend(_p(q), _p(kv), kv_dt, _p(kv_scale), N_cap, _p(sel), k, _p(n_elig),
                     _p(win), win_dt, W_buf, _p(win_begin), _p(win_len), _p(sink), float(tau),
                     B, Tq, Hq, D, _p(o), _p(lse), _p(v), _p(v_scale), _p(win_v))
    return o, lse


def num_threads() -> int:
    return lib().orc_num_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (results do not depend on it)."""
    lib().orc_set_threads(int(n))
