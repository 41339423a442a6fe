"""Python binding of liblca.so, the MI355X (gfx950) CSA/HCA hot-path library.

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch tensors on the GPU (PyTorch provides device memory and the
current stream); each wrapper passes their data pointers to the C ABI declared
in include/lca.h and raises LcaError when the library reports an error.  If
the built library is missing, importing works but every call raises.

Storage types: F32 (torch.float32), BF16 (torch.bfloat16), FP8E4M3 (uint8 codes
+ float32 scale per 64 elements), MXFP4 (uint8, two E2M1 codes per byte +
uint8 E8M0 scale per 32 elements).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblca.so")

F32, BF16, FP8E4M3, MXFP4 = 0, 1, 2, 3
STATUS = {0: "LCA_OK", 1: "LCA_EINVAL", 2: "LCA_ENOTSUP", 3: "LCA_EHIP", 4: "LCA_EWORKSPACE"}

EXPORTS = ["lca_abi_version", "lca_last_error", "lca_csa_compress", "lca_hca_compress", "lca_compress_batch",
           "lca_lightning_index_topk", "lca_index_topk_ws", "lca_sparse_mqa_attend",
           "lca_hca_attend", "lca_attend_batch", "lca_attend_ws", "lca_decode_step", "lca_decode_append", "lca_window_attend",
           "lca_decode_loop_step", "lca_attend_separate_v", "lca_decode_step_events", "lca_decode_step_noalloc"]
MAX_STEP_LAUNCHES = 8
MAX_COMPRESS_JOBS = 8
MAX_ATTEND_JOBS = 4
MAX_APPEND_JOBS = 8


class CompressJob(ctypes.Structure):
    """lca_compress_job: the argument list of one compress call."""
    _fields_ = [("x", ctypes.c_void_p), ("x_dt", ctypes.c_int32), ("x_rows", ctypes.c_int64),
                ("gate", ctypes.c_void_p), ("pos_bias", ctypes.c_void_p), ("m", ctypes.c_int32),
                ("x_tok0", ctypes.c_void_p), ("nblk", ctypes.c_void_p), ("dst_row0", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("nblk_max", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dst", ctypes.c_void_p), ("dst_dt", ctypes.c_int32), ("dst_scale", ctypes.c_void_p),
                ("dst_rows", ctypes.c_int64), ("pooled", ctypes.c_void_p), ("gate_pc", ctypes.c_int32),
                ("overlap", ctypes.c_int32)]


class LcaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load liblca.so (no GPU needed) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LcaError(3, f"liblca.so not built at {path}; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    L.lca_abi_version.restype = i32
    L.lca_abi_version.argtypes = []
    L.lca_last_error.restype = ctypes.c_char_p
    L.lca_last_error.argtypes = []
    comp = [vp, i32, i64, vp, vp, i32, vp, vp, vp, i32, i32, i32, vp, i32, vp, i64, vp, vp]
    for name in ("lca_csa_compress", "lca_hca_compress"):
        getattr(L, name).restype = i32
        getattr(L, name).argtypes = comp
    L.lca_decode_step.restype = i32
    L.lca_decode_step.argtypes = [ctypes.POINTER(CompressJob), i32, ctypes.POINTER(IndexJob),
                                  ctypes.POINTER(AttendJob), i32, vp]
    L.lca_decode_step_noalloc.restype = i32
    L.lca_decode_step_noalloc.argtypes = [ctypes.POINTER(CompressJob), i32, ctypes.POINTER(IndexJob),
                                          ctypes.POINTER(AttendJob), i32, vp]
    L.lca_decode_step_events.restype = i32
    L.lca_decode_step_events.argtypes = [ctypes.POINTER(CompressJob), i32, ctypes.POINTER(IndexJob),
                                         ctypes.POINTER(AttendJob), i32, ctypes.POINTER(vp), i32,
                                         ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(i32), vp]
    L.lca_decode_loop_step.restype = i32
    L.lca_decode_loop_step.argtypes = [ctypes.POINTER(AppendJob), i32, ctypes.POINTER(CompressJob), i32,
                                       ctypes.POINTER(IndexJob), ctypes.POINTER(AttendJob), i32, vp]
    L.lca_decode_append.restype = i32
    L.lca_decode_append.argtypes = [ctypes.POINTER(AppendJob), i32, vp]
    L.lca_attend_batch.restype = i32
    L.lca_attend_batch.argtypes = [ctypes.POINTER(AttendJob), i32, vp]
    L.lca_compress_batch.restype = i32
    L.lca_compress_batch.argtypes = [ctypes.POINTER(CompressJob), i32, vp]
    L.lca_lightning_index_topk.restype = i32
    L.lca_lightning_index_topk.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i64,
                                           i32, vp, vp, vp, sz, vp]
    L.lca_index_topk_ws.restype = sz
    L.lca_index_topk_ws.argtypes = [i32, i32, i32, i32, i64, i32]
    L.lca_sparse_mqa_attend.restype = i32
    L.lca_sparse_mqa_attend.argtypes = [vp, i32, vp, i32, vp, i64, vp, i32, vp, i32, i64, vp, vp, vp,
                                        f32, i32, i32, i32, i32, vp, i32, vp, vp, sz, vp]
    L.lca_hca_attend.restype = i32
    L.lca_hca_attend.argtypes = [vp, i32, vp, i32, vp, i64, vp, vp, i32, i64, vp, vp, vp, f32, i32,
                                 i32, i32, i32, vp, i32, vp, vp, sz, vp]
    L.lca_attend_ws.restype = sz
    L.lca_attend_ws.argtypes = [i32, i32, i32, i32, i64, i64]
    L.lca_attend_separate_v.restype = i32
    L.lca_attend_separate_v.argtypes = [i32, vp, i32, vp, vp, i32, vp, vp, i64, vp, i32, vp, vp, vp, i32, i64, vp, vp,
                                        vp, f32, i32, i32, i32, i32, vp, i32, vp, vp, sz, vp]
    L.lca_window_attend.restype = i32
    L.lca_window_attend.argtypes = [vp, i32, vp, i32, i64, vp, vp, vp, f32, i32, i32, i32, i32, vp, i32, vp, vp, sz,
                                    vp]
    _lib = L
    return L


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int):
    if status != 0:
        raise LcaError(status, load().lca_last_error().decode())


def dtype_of(t, scale=None) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.uint8:
        if scale is None:
            raise ValueError("uint8 storage needs its scale tensor")
        return FP8E4M3 if scale.dtype == torch.float32 else MXFP4
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


def abi_version() -> int:
    return load().lca_abi_version()


# ---------------------------------------------------------------------------
def _compress(fn, x, gate, pos_bias, m, x_tok0, nblk, dst_row0, nblk_max, dst, dst_dt,
              dst_scale=None, pooled=None, stream=None):
    B, x_rows, D = x.shape
    _check(fn(_p(x), dtype_of(x), x_rows, _p(gate), _p(pos_bias), int(m), _p(x_tok0), _p(nblk),
              _p(dst_row0), B, int(nblk_max), D, _p(dst), int(dst_dt), _p(dst_scale),
              dst.shape[1], _p(pooled), _stream(stream)))


def csa_compress(x, gate, pos_bias, m, x_tok0, nblk, dst_row0, nblk_max, dst, dst_dt,
                 dst_scale=None, pooled=None, stream=None):
    """Pool blocks of m raw tokens into cache rows (see lca_csa_compress).
    x [B, x_rows, D] f32/bf16; gate [B, x_rows] f32; pos_bias [m] f32;
    x_tok0/nblk int32 [B], dst_row0 int64 [B] on the device; dst [B, rows, D or D/2]."""
    _compress(load().lca_csa_compress, x, gate, pos_bias, m, x_tok0, nblk, dst_row0, nblk_max,
              dst, dst_dt, dst_scale, pooled, stream)


def hca_compress(x, gate, pos_bias, m, x_tok0, nblk, dst_row0, nblk_max, dst, dst_dt,
                 dst_scale=None, pooled=None, stream=None):
    """As csa_compress, for m' up to 1024 (see lca_hca_compress)."""
    _compress(load().lca_hca_compress, x, gate, pos_bias, m, x_tok0, nblk, dst_row0, nblk_max,
              dst, dst_dt, dst_scale, pooled, stream)


def compress_job(x, gate, pos_bias, m, x_tok0, nblk, dst_row0, nblk_max, dst, dst_dt, dst_scale=None,
                 pooled=None, overlap=0) -> CompressJob:
    """One job of compress_batch, with the arguments of csa_compress / hca_compress; a gate of
    shape [B, x_rows, D] selects per-channel gates (pos_bias [m + overlap, D]), overlap > 0
    overlapping blocks (see lca_compress_batch).  The job holds references to its tensors, so
    they stay allocated while the job object is alive (keep it until the call)."""
    B, x_rows, D = x.shape
    ptr = lambda t: None if t is None else t.data_ptr()
    job = CompressJob(ptr(x), dtype_of(x), x_rows, ptr(gate), ptr(pos_bias), int(m), ptr(x_tok0), ptr(nblk),
                      ptr(dst_row0), B, int(nblk_max), D, ptr(dst), int(dst_dt), ptr(dst_scale), dst.shape[1],
                      ptr(pooled), 1 if gate.dim() == 3 else 0, int(overlap))
    job._keep = (x, gate, pos_bias, x_tok0, nblk, dst_row0, dst, dst_scale, pooled)
    return job


def compress_batch(jobs, stream=None):
    """Several compress calls in one launch (see lca_compress_batch); jobs from compress_job(),
    or a ctypes array of them built once (e.g. for a step that is issued many times)."""
    arr = jobs if isinstance(jobs, ctypes.Array) else (CompressJob * len(jobs))(*jobs)
    _check(load().lca_compress_batch(arr, len(arr), _stream(stream)))


class AttendJob(ctypes.Structure):
    """lca_attend_job: the argument list of one sparse_mqa_attend / hca_attend call."""
    _fields_ = [("sparse", ctypes.c_int32), ("q", ctypes.c_void_p), ("q_dt", ctypes.c_int32),
                ("kv", ctypes.c_void_p), ("kv_dt", ctypes.c_int32), ("kv_scale", ctypes.c_void_p),
                ("N_cap", ctypes.c_int64), ("idx", ctypes.c_void_p), ("k", ctypes.c_int32),
                ("n_elig", ctypes.c_void_p), ("win", ctypes.c_void_p), ("win_dt", ctypes.c_int32),
                ("W_buf", ctypes.c_int64), ("win_begin", ctypes.c_void_p), ("win_len", ctypes.c_void_p),
                ("sink", ctypes.c_void_p), ("scale", ctypes.c_float), ("B", ctypes.c_int32), ("Tq", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("D", ctypes.c_int32), ("out", ctypes.c_void_p), ("out_dt", ctypes.c_int32),
                ("lse", ctypes.c_void_p), ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


def attend_job(sparse, q, kv, kv_scale, idx_or_n, win, win_begin, win_len, sink, scale, out, lse=None,
               ws=None) -> AttendJob:
    """One job of attend_batch: the arguments of sparse_mqa_attend (sparse=True, idx) or
    hca_attend (sparse=False, n_elig); kv=None with sparse=True and idx_or_n=None is a
    window_attend job.  The job holds references to its tensors, so they stay allocated while
    the job object is alive (keep it until attend_batch has been called)."""
    B, Tq, Hq, D = q.shape
    ptr = lambda t: None if t is None else t.data_ptr()
    if kv is None and not (sparse and idx_or_n is None):
        raise ValueError("kv=None describes a window-only job: sparse=True, idx_or_n=None")
    job = AttendJob(1 if sparse else 0, ptr(q), dtype_of(q), ptr(kv), BF16 if kv is None else dtype_of(kv, kv_scale),
                    ptr(kv_scale), 0 if kv is None else kv.shape[1], ptr(idx_or_n) if sparse else None,
                    (0 if idx_or_n is None else idx_or_n.shape[-1]) if sparse else 0,
                    None if sparse else ptr(idx_or_n), ptr(win), dtype_of(win), win.shape[1], ptr(win_begin),
                    ptr(win_len), ptr(sink), float(scale), B, Tq, Hq, D, ptr(out), dtype_of(out), ptr(lse),
                    ptr(ws), 0 if ws is None else ws.numel() * ws.element_size())
    job._keep = (q, kv, kv_scale, idx_or_n, win, win_begin, win_len, sink, out, lse, ws)
    return job


def attend_batch(jobs, stream=None):
    """Several attention calls in one launch (see lca_attend_batch); jobs from attend_job(),
    or a ctypes array of them built once."""
    arr = jobs if isinstance(jobs, ctypes.Array) else (AttendJob * len(jobs))(*jobs)
    _check(load().lca_attend_batch(arr, len(arr), _stream(stream)))


class IndexJob(ctypes.Structure):
    """lca_index_job: the argument list of one lightning_index_topk call."""
    _fields_ = [("qi", ctypes.c_void_p), ("qi_dt", ctypes.c_int32), ("qi_scale", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("ki", ctypes.c_void_p), ("ki_dt", ctypes.c_int32),
                ("ki_scale", ctypes.c_void_p), ("n_elig", ctypes.c_void_p), ("B", ctypes.c_int32),
                ("Tq", ctypes.c_int32), ("H_I", ctypes.c_int32), ("d_I", ctypes.c_int32), ("N_cap", ctypes.c_int64),
                ("k", ctypes.c_int32), ("idx_out", ctypes.c_void_p), ("score_out", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


def index_job(qi, qi_scale, w, ki, ki_scale, n_elig, k, idx_out, ws, score_out=None) -> IndexJob:
    """The indexer part of decode_step, with the arguments of lightning_index_topk (the job
    keeps its tensors alive while it is)."""
    B, Tq, H = qi.shape[0], qi.shape[1], qi.shape[2]
    dt = F32 if qi_scale is None else MXFP4
    d = qi.shape[3] if dt == F32 else qi.shape[3] * 2
    ptr = lambda t: None if t is None else t.data_ptr()
    job = IndexJob(ptr(qi), dt, ptr(qi_scale), ptr(w), ptr(ki), dt, ptr(ki_scale), ptr(n_elig), B, Tq, H, d,
                   ki.shape[1], int(k), ptr(idx_out), ptr(score_out), ptr(ws),
                   0 if ws is None else ws.numel() * ws.element_size())
    job._keep = (qi, qi_scale, w, ki, ki_scale, n_elig, idx_out, ws, score_out)
    return job


def decode_step(cjobs, ijob, ajobs, stream=None):
    """One decode step (see lca_decode_step): compress jobs, the indexer job (None: no
    indexer), attention jobs; job lists may be prebuilt ctypes arrays."""
    ca = cjobs if isinstance(cjobs, ctypes.Array) else (CompressJob * max(1, len(cjobs)))(*cjobs)
    aa = ajobs if isinstance(ajobs, ctypes.Array) else (AttendJob * max(1, len(ajobs)))(*ajobs)
    ij = None if ijob is None else ctypes.byref(ijob)
    _check(load().lca_decode_step(ca, len(cjobs), ij, aa, len(ajobs), _stream(stream)))


def decode_step_noalloc(cjobs, ijob, ajobs, stream=None):
    """decode_step with every workspace taken from the library's per-GPU
    scratch (see lca_decode_step_noalloc); the jobs' ws fields are ignored."""
    ca = cjobs if isinstance(cjobs, ctypes.Array) else (CompressJob * max(1, len(cjobs)))(*cjobs)
    aa = ajobs if isinstance(ajobs, ctypes.Array) else (AttendJob * max(1, len(ajobs)))(*ajobs)
    ij = None if ijob is None else ctypes.byref(ijob)
    _check(load().lca_decode_step_noalloc(ca, len(cjobs), ij, aa, len(ajobs), _stream(stream)))


def decode_step_events(cjobs, ijob, ajobs, events, stream=None):
    """decode_step with HIP events recorded around its launches (see
    lca_decode_step_events).  events: MAX_STEP_LAUNCHES + 1 torch.cuda.Event
    objects already created (recorded once); returns the kernel names of the
    launches made, launch i between events[i] and events[i + 1]."""
    ca = cjobs if isinstance(cjobs, ctypes.Array) else (CompressJob * max(1, len(cjobs)))(*cjobs)
    aa = ajobs if isinstance(ajobs, ctypes.Array) else (AttendJob * max(1, len(ajobs)))(*ajobs)
    ij = None if ijob is None else ctypes.byref(ijob)
    ev = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    names = (ctypes.c_char_p * MAX_STEP_LAUNCHES)()
    n = ctypes.c_int32(0)
    _check(load().lca_decode_step_events(ca, len(cjobs), ij, aa, len(ajobs), ev, len(events), names,
                                         ctypes.byref(n), _stream(stream)))
    return [names[i].decode() for i in range(n.value)]


class AppendJob(ctypes.Structure):
    """lca_append_job: one raw-token stream of decode_append."""
    _fields_ = [("x_new", ctypes.c_void_p), ("x_dt", ctypes.c_int32), ("g_new", ctypes.c_void_p),
                ("ring", ctypes.c_void_p), ("gring", ctypes.c_void_p), ("R", ctypes.c_int64),
                ("len", ctypes.c_void_p), ("m", ctypes.c_int32), ("W", ctypes.c_int32),
                ("x_tok0", ctypes.c_void_p), ("nblk", ctypes.c_void_p), ("dst_row0", ctypes.c_void_p),
                ("n_elig", ctypes.c_void_p), ("win_begin", ctypes.c_void_p), ("win_len", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("D", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("gate_pc", ctypes.c_int32)]


def append_job(x_new, ring, length, m=0, W=0, g_new=None, gring=None, x_tok0=None, nblk=None, dst_row0=None,
               n_elig=None, win_begin=None, win_len=None, overlap=0) -> AppendJob:
    """One stream of decode_append: x_new [B, D] new tokens, ring [B, 2R, D] (gring [B, 2R]),
    length [B] int64 tokens so far; the outputs are the step arguments named in lca.h (the job
    keeps its tensors alive while it is)."""
    B, R2, D = ring.shape
    ptr = lambda t: None if t is None else t.data_ptr()
    job = AppendJob(ptr(x_new), dtype_of(x_new), ptr(g_new), ptr(ring), ptr(gring), R2 // 2, ptr(length), int(m),
                    int(W), ptr(x_tok0), ptr(nblk), ptr(dst_row0), ptr(n_elig), ptr(win_begin), ptr(win_len), B, D,
                    int(overlap), 1 if gring is not None and gring.dim() == 3 else 0)
    job._keep = (x_new, g_new, ring, gring, length, x_tok0, nblk, dst_row0, n_elig, win_begin, win_len)
    return job


def decode_append(jobs, stream=None):
    """Append one token per sequence to each stream (see lca_decode_append); jobs from
    append_job(), or a ctypes array of them built once."""
    arr = jobs if isinstance(jobs, ctypes.Array) else (AppendJob * len(jobs))(*jobs)
    _check(load().lca_decode_append(arr, len(arr), _stream(stream)))


def decode_loop_step(ajobs_append, cjobs, ijob, ajobs, stream=None):
    """decode_append(ajobs_append) then decode_step(cjobs, ijob, ajobs) in one call, the appends
    inside the compress launch (see lca_decode_loop_step); lists or prebuilt ctypes arrays."""
    pa = ajobs_append if isinstance(ajobs_append, ctypes.Array) else \
        (AppendJob * max(1, len(ajobs_append)))(*ajobs_append)
    ca = cjobs if isinstance(cjobs, ctypes.Array) else (CompressJob * max(1, len(cjobs)))(*cjobs)
    aa = ajobs if isinstance(ajobs, ctypes.Array) else (AttendJob * max(1, len(ajobs)))(*ajobs)
    ij = None if ijob is None else ctypes.byref(ijob)
    _check(load().lca_decode_loop_step(pa, len(ajobs_append), ca, len(cjobs), ij, aa, len(ajobs), _stream(stream)))


# ---------------------------------------------------------------------------
def index_topk_ws(B, Tq, H_I, d_I, N_cap, k) -> int:
    return load().lca_index_topk_ws(B, Tq, H_I, d_I, N_cap, k)


def lightning_index_topk(qi, qi_scale, w, ki, ki_scale, n_elig, k, idx_out, ws, score_out=None,
                         H_I=None, d_I=None, stream=None):
    """qi [B, Tq, H_I, d_I] f32, or uint8 [B, Tq, H_I, d_I/2] + qi_scale E8M0;
    w [B, Tq, H_I] f32; ki [B, N_cap, d_I] f32 or uint8 [B, N_cap, d_I/2] + ki_scale;
    n_elig int32 [B, Tq]; idx_out int32 [B, Tq, k]; ws uint8 workspace."""
    B, Tq = qi.shape[0], qi.shape[1]
    H = qi.shape[2] if H_I is None else H_I
    dt = F32 if qi_scale is None else MXFP4
    d = (qi.shape[3] if dt == F32 else qi.shape[3] * 2) if d_I is None else d_I
    N_cap = ki.shape[1]
    _check(load().lca_lightning_index_topk(
        _p(qi), dt, _p(qi_scale), _p(w), _p(ki), dt, _p(ki_scale), _p(n_elig), B, Tq, H, d, N_cap,
        int(k), _p(idx_out), _p(score_out), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


# ---------------------------------------------------------------------------
def attend_ws(B, Tq, Hq, D, n_kv_max, W_buf) -> int:
    return load().lca_attend_ws(B, Tq, Hq, D, n_kv_max, W_buf)


def sparse_mqa_attend(q, kv, kv_scale, idx, win, win_begin, win_len, sink, scale, out, lse=None,
                      ws=None, stream=None):
    """q [B,Tq,Hq,D] f32/bf16; kv [B,N_cap,D] f32/bf16/uint8(+kv_scale f32 [B,N_cap,D/64]);
    idx int32 [B,Tq,k]; win [B,W_buf,D]; win_begin/win_len int32 [B,Tq]; sink f32 [Hq];
    out [B,Tq,Hq,D] f32/bf16; lse optional f32 [B,Tq,Hq]."""
    B, Tq, Hq, D = q.shape
    k = idx.shape[-1]
    _check(load().lca_sparse_mqa_attend(
        _p(q), dtype_of(q), _p(kv), dtype_of(kv, kv_scale), _p(kv_scale), kv.shape[1], _p(idx), k,
        _p(win), dtype_of(win), win.shape[1], _p(win_begin), _p(win_len), _p(sink), float(scale),
        B, Tq, Hq, D, _p(out), dtype_of(out), _p(lse), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def hca_attend(q, kv, kv_scale, n_elig, win, win_begin, win_len, sink, scale, out, lse=None,
               ws=None, stream=None):
    """As sparse_mqa_attend, attending densely over entries j < n_elig [B,Tq]."""
    B, Tq, Hq, D = q.shape
    _check(load().lca_hca_attend(
        _p(q), dtype_of(q), _p(kv), dtype_of(kv, kv_scale), _p(kv_scale), kv.shape[1], _p(n_elig),
        _p(win), dtype_of(win), win.shape[1], _p(win_begin), _p(win_len), _p(sink), float(scale),
        B, Tq, Hq, D, _p(out), dtype_of(out), _p(lse), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def window_attend(q, win, win_begin, win_len, sink, scale, out, lse=None, ws=None, stream=None):
    """Attention over the window rows and the sink only (see lca_window_attend)."""
    B, Tq, Hq, D = q.shape
    _check(load().lca_window_attend(
        _p(q), dtype_of(q), _p(win), dtype_of(win), win.shape[1], _p(win_begin), _p(win_len), _p(sink),
        float(scale), B, Tq, Hq, D, _p(out), dtype_of(out), _p(lse), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def attend_separate_v(sparse, q, k, v, k_scale, v_scale, idx_or_n, win_k, win_v, win_begin, win_len, sink, scale,
                      out, lse=None, ws=None, stream=None):
    """sparse_mqa_attend (sparse=True, idx) or hca_attend (sparse=False, n_elig) with separate
    key and value vectors (see lca_attend_separate_v)."""
    B, Tq, Hq, D = q.shape
    _check(load().lca_attend_separate_v(
        1 if sparse else 0, _p(q), dtype_of(q), _p(k), _p(v), dtype_of(k, k_scale), _p(k_scale), _p(v_scale),
        k.shape[1], _p(idx_or_n) if sparse else None, idx_or_n.shape[-1] if sparse else 0,
        None if sparse else _p(idx_or_n), _p(win_k), _p(win_v), dtype_of(win_k), win_k.shape[1], _p(win_begin),
        _p(win_len), _p(sink), float(scale), B, Tq, Hq, D, _p(out), dtype_of(out), _p(lse), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))
