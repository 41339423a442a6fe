"""C-ABI contract tests that need no GPU: the library loads, exports every
entry point that include/lca.h declares, and rejects invalid arguments with
the documented status before touching the GPU."""
import ctypes
import os
import re

import pytest

import long_context_attention_13_amd as lca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lca.h")

FAKE = 0x10000      # a non-null, aligned address; never dereferenced on these paths


def header_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(lca_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    return lca.load()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert set(names) == set(lca.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version(L):
    assert L.lca_abi_version() == 3


def compress(L, **kw):
    a = dict(x=FAKE, x_dt=lca.F32, x_rows=64, gate=FAKE, pos_bias=FAKE, m=4, x_tok0=FAKE, nblk=FAKE,
             dst_row0=FAKE, B=2, nblk_max=16, D=128, dst=FAKE, dst_dt=lca.F32, dst_scale=None,
             dst_rows=16, pooled=None, stream=None)
    a.update(kw)
    return L.lca_csa_compress(*a.values())


def test_compress_validation(L):
    assert compress(L, x=None) == 1
    assert b"x must be" in L.lca_last_error()
    assert compress(L, x=FAKE + 4) == 1              # misaligned
    assert compress(L, m=0) == 2
    assert compress(L, m=65) == 2                    # csa_compress: m <= 64
    assert compress(L, D=96) == 2
    assert compress(L, x_dt=lca.FP8E4M3) == 2
    assert compress(L, nblk_max=17) == 1             # exceeds x_rows / m and dst_rows
    assert compress(L, dst_dt=lca.FP8E4M3) == 1      # FP8 needs a scale pointer
    assert compress(L, dst_dt=lca.F32, dst_scale=FAKE) == 1
    assert compress(L, B=0) == 0                     # nothing to do, no GPU touched
    assert L.lca_last_error() == b""
    args = dict(x=None, x_dt=lca.F32, x_rows=4096, gate=FAKE, pos_bias=FAKE, m=200, x_tok0=FAKE,
                nblk=FAKE, dst_row0=FAKE, B=1, nblk_max=8, D=128, dst=FAKE, dst_dt=lca.F32,
                dst_scale=None, dst_rows=8, pooled=None, stream=None)
    assert L.lca_hca_compress(*args.values()) == 1   # m=200 accepted; fails on the null x
    args["m"] = 1025
    assert L.lca_hca_compress(*args.values()) == 2


def index(L, **kw):
    a = dict(qi=FAKE, qi_dt=lca.MXFP4, qi_scale=FAKE, w=FAKE, ki=FAKE, ki_dt=lca.MXFP4, ki_scale=FAKE,
             n_elig=FAKE, B=1, Tq=1, H_I=8, d_I=128, N_cap=1024, k=64, idx_out=FAKE, score_out=None,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.lca_lightning_index_topk(*a.values())


def test_index_validation(L):
    assert index(L, k=0) == 1
    assert index(L, k=2049) == 1
    assert index(L, H_I=17) == 2
    assert index(L, d_I=96) == 2
    assert index(L, ki_dt=lca.F32) == 2
    assert index(L, qi_dt=lca.BF16, ki_dt=lca.BF16) == 2
    assert index(L, qi_dt=lca.F32, ki_dt=lca.F32) == 1        # F32 must not pass scales
    f32 = dict(qi_dt=lca.F32, ki_dt=lca.F32, qi_scale=None, ki_scale=None, d_I=64)
    assert index(L, H_I=17, **f32) == 2                        # F32: the kernels stage 16 head weights
    assert index(L, ws=None) == 4
    assert index(L, ws_bytes=16) == 4
    assert b"workspace" in L.lca_last_error()
    assert index(L, idx_out=None) == 1
    assert index(L, B=0) == 0
    need = L.lca_index_topk_ws(4, 1, 8, 128, 262144, 1024)
    assert 0 < need < 64 << 20


def attend(L, fn="lca_sparse_mqa_attend", **kw):
    a = dict(q=FAKE, q_dt=lca.BF16, kv=FAKE, kv_dt=lca.FP8E4M3, kv_scale=FAKE, N_cap=1024, idx=FAKE,
             k=64, win=FAKE, win_dt=lca.BF16, W_buf=128, win_begin=FAKE, win_len=FAKE, sink=FAKE,
             scale=0.088, B=1, Tq=1, Hq=64, D=128, out=FAKE, out_dt=lca.BF16, lse=None, ws=FAKE,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    if fn == "lca_hca_attend":
        a.pop("k")
        keys = list(a)
        keys[keys.index("idx")] = "n_elig"
        a = dict(zip(keys, a.values()))
    return getattr(L, fn)(*a.values())


def test_attend_validation(L):
    assert attend(L, D=64) == 2
    assert attend(L, Hq=8) == 2
    assert attend(L, kv_dt=lca.MXFP4) == 2
    assert attend(L, k=2049) == 1
    assert attend(L, kv_scale=None) == 1
    assert attend(L, kv_dt=lca.BF16) == 1                    # scale given for non-FP8
    assert attend(L, k=1024, ws=None) == 4                  # 1024 + 128 items: split partials
    assert attend(L, k=1024, ws_bytes=100) == 4
    assert attend(L, fn="lca_hca_attend", idx=None) == 1     # n_elig is required
    assert attend(L, fn="lca_hca_attend", q=None) == 1
    assert attend(L, B=0) == 0
    assert L.lca_attend_ws(4, 1, 64, 128, 8192, 128) > 0
    assert L.lca_attend_ws(1, 8192, 64, 128, 1024, 8319) == 0   # enough rows: no splits


def test_errors_are_thread_local(L):
    import threading
    assert compress(L, D=96) == 2
    seen = []
    t = threading.Thread(target=lambda: seen.append(L.lca_last_error()))
    t.start()
    t.join()
    assert seen == [b""]
    assert L.lca_last_error() != b""


def batch_job(**kw):
    a = dict(x=FAKE, x_dt=lca.BF16, x_rows=256, gate=FAKE, pos_bias=FAKE, m=4, x_tok0=FAKE, nblk=FAKE,
             dst_row0=FAKE, B=2, nblk_max=1, D=128, dst=FAKE, dst_dt=lca.FP8E4M3, dst_scale=FAKE,
             dst_rows=16, pooled=None)
    a.update(kw)
    return lca.CompressJob(**a)


def compress_batch(L, jobs, n=None):
    arr = (lca.CompressJob * max(1, len(jobs)))(*jobs)
    return L.lca_compress_batch(arr, len(jobs) if n is None else n, None)


def test_compress_batch_validation(L):
    ok3 = [batch_job(), batch_job(dst_dt=lca.MXFP4), batch_job(m=128, x_rows=256)]
    assert compress_batch(L, [batch_job(B=0)] * 3) == 0          # nothing to do, no GPU touched
    assert compress_batch(L, ok3, n=0) == 1
    assert compress_batch(L, ok3 * 3, n=9) == 1                   # more than LCA_MAX_COMPRESS_JOBS
    assert L.lca_compress_batch(None, 1, None) == 1
    bad = list(ok3)
    bad[1] = batch_job(m=2048)                                    # m above 1024
    assert compress_batch(L, bad) == 2
    assert b"job 1" in L.lca_last_error()
    bad[1] = batch_job(dst=None)
    assert compress_batch(L, bad) == 1
    bad[1] = batch_job(D=64)                                      # D differs from job 0
    assert compress_batch(L, bad) == 2
    bad[1] = batch_job(x_dt=lca.F32)                              # x_dt differs from job 0
    assert compress_batch(L, bad) == 2
    bad[2] = batch_job(nblk_max=100)                              # nblk_max*m exceeds x_rows
    assert compress_batch(L, bad) in (1, 2)


def attend_job(**kw):
    a = dict(sparse=1, q=FAKE, q_dt=lca.BF16, kv=FAKE, kv_dt=lca.FP8E4M3, kv_scale=FAKE, N_cap=1024, idx=FAKE,
             k=64, n_elig=None, win=FAKE, win_dt=lca.BF16, W_buf=128, win_begin=FAKE, win_len=FAKE, sink=FAKE,
             scale=0.088, B=1, Tq=1, Hq=64, D=128, out=FAKE, out_dt=lca.BF16, lse=None, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(kw)
    return lca.AttendJob(*a.values())


def attend_batch(L, jobs, n=None):
    arr = (lca.AttendJob * max(1, len(jobs)))(*jobs)
    return L.lca_attend_batch(arr, len(jobs) if n is None else n, None)


def test_attend_batch_validation(L):
    dense = dict(sparse=0, idx=None, k=0, n_elig=FAKE)
    assert attend_batch(L, [attend_job(B=0), attend_job(B=0, **dense)]) == 0   # nothing to do
    assert attend_batch(L, [attend_job()], n=0) == 1
    assert attend_batch(L, [attend_job()] * 5) == 1                           # more than LCA_MAX_ATTEND_JOBS
    assert L.lca_attend_batch(None, 1, None) == 1
    assert attend_batch(L, [attend_job(), attend_job(sparse=2)]) == 1
    assert attend_batch(L, [attend_job(), attend_job(idx=None)]) == 1
    assert b"job 1" in L.lca_last_error()
    assert attend_batch(L, [attend_job(), attend_job(n_elig=None, **{k: v for k, v in dense.items()
                                                                     if k != "n_elig"})]) == 1
    assert attend_batch(L, [attend_job(), attend_job(Hq=32)]) == 2          # Hq differs from job 0
    assert attend_batch(L, [attend_job(), attend_job(kv_dt=lca.BF16, kv_scale=None)]) == 2
    assert attend_batch(L, [attend_job(q_dt=lca.F32)]) == 2                  # not the bf16 MFMA path
    # the chunked-prefill dense shape (many rows, no split) stays with lca_hca_attend
    assert attend_batch(L, [attend_job(Tq=8192, W_buf=8319, N_cap=2048, **dense)]) == 2
    assert attend_batch(L, [attend_job(k=1024, ws=None)]) == 4               # split partials need workspace


def index_job(**kw):
    a = dict(qi=FAKE, qi_dt=lca.MXFP4, qi_scale=FAKE, w=FAKE, ki=FAKE, ki_dt=lca.MXFP4, ki_scale=FAKE, n_elig=FAKE,
             B=1, Tq=1, H_I=8, d_I=128, N_cap=1024, k=64, idx_out=FAKE, score_out=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lca.IndexJob(*a.values())


def decode_step(L, cjobs, ij, ajobs, nc=None, na=None):
    ca = (lca.CompressJob * max(1, len(cjobs)))(*cjobs)
    aa = (lca.AttendJob * max(1, len(ajobs)))(*ajobs)
    return L.lca_decode_step(ca, len(cjobs) if nc is None else nc, None if ij is None else ctypes.byref(ij), aa,
                             len(ajobs) if na is None else na, None)


def test_decode_step_validation(L):
    assert decode_step(L, [], index_job(B=0), []) == 0                       # nothing to do
    assert decode_step(L, [batch_job(B=0)], index_job(B=0), [attend_job(B=0)]) == 0
    assert decode_step(L, [], None, []) == 0                                  # no indexer
    assert decode_step(L, [batch_job(B=0)], None, [attend_job(B=0)]) == 0
    assert decode_step(L, [batch_job()] * 9, index_job(B=0), []) == 1
    assert decode_step(L, [], index_job(B=0), [attend_job()] * 5) == 1
    assert decode_step(L, [], index_job(k=0), []) == 1
    assert b"index job" in L.lca_last_error()
    assert decode_step(L, [batch_job(m=2048)], index_job(B=0), []) == 2
    assert b"compress job 0" in L.lca_last_error()
    assert decode_step(L, [], index_job(B=0), [attend_job(), attend_job(Hq=32)]) == 2
    assert b"attention job 1" in L.lca_last_error()
    assert decode_step(L, [], index_job(ws=None), []) == 4
    # a dense job that would write the indexer's output while the scan runs
    dense = attend_job(sparse=0, idx=None, k=0, n_elig=FAKE, out=FAKE + 4096)
    assert decode_step(L, [], index_job(idx_out=FAKE + 4096), [dense]) == 1
    assert b"index job writes" in L.lca_last_error()


def test_decode_step_events_validation(L):
    """Argument checks of the measurement form of the decode step (no GPU:
    every case fails or has nothing to launch before any event is touched)."""
    n = ctypes.c_int32(-1)
    names = (ctypes.c_char_p * lca.MAX_STEP_LAUNCHES)()
    ev = (ctypes.c_void_p * (lca.MAX_STEP_LAUNCHES + 1))(*([FAKE] * (lca.MAX_STEP_LAUNCHES + 1)))
    ca = (lca.CompressJob * 1)(batch_job(B=0))
    aa = (lca.AttendJob * 1)(attend_job(B=0))
    call = lambda evs, nev, nl, ij=index_job(k=0): L.lca_decode_step_events(
        ca, 1, ctypes.byref(ij), aa, 1, evs, nev, names, nl, None)
    assert call(None, lca.MAX_STEP_LAUNCHES + 1, ctypes.byref(n)) == 1
    assert call(ev, lca.MAX_STEP_LAUNCHES, ctypes.byref(n)) == 1               # too few events
    assert b"event handles" in L.lca_last_error()
    assert call(ev, lca.MAX_STEP_LAUNCHES + 1, None) == 1
    ev_null = (ctypes.c_void_p * (lca.MAX_STEP_LAUNCHES + 1))(*([FAKE] * lca.MAX_STEP_LAUNCHES + [None]))
    assert call(ev_null, lca.MAX_STEP_LAUNCHES + 1, ctypes.byref(n)) == 1
    assert b"events[8]" in L.lca_last_error()
    assert call(ev, lca.MAX_STEP_LAUNCHES + 1, ctypes.byref(n)) == 1           # the index job's k = 0
    assert b"index job" in L.lca_last_error() and n.value == -1


def test_decode_step_noalloc_validation(L):
    """The allocation-free step validates as the step does and rejects a step
    whose workspaces exceed the library's scratch before touching the GPU."""
    ca = (lca.CompressJob * 1)(batch_job(B=0))
    aa = (lca.AttendJob * 1)(attend_job(B=0))
    call = lambda ij, na=1: L.lca_decode_step_noalloc(ca, 1, None if ij is None else ctypes.byref(ij), aa, na, None)
    big = index_job(B=256, N_cap=1 << 24, k=1024)
    assert L.lca_index_topk_ws(256, 1, 8, 128, 1 << 24, 1024) > 64 << 20
    assert call(big) == 4
    assert b"scratch" in L.lca_last_error()
    assert call(index_job(k=0)) == 1
    assert b"index job" in L.lca_last_error()
    assert call(None, na=5) == 1
    assert call(index_job(B=0)) == 0                 # nothing to do: no GPU call


def append_job(**kw):
    a = dict(x_new=FAKE, x_dt=lca.BF16, g_new=FAKE, ring=FAKE, gring=FAKE, R=256, len=FAKE, m=4, W=128,
             x_tok0=FAKE, nblk=FAKE, dst_row0=FAKE, n_elig=FAKE, win_begin=FAKE, win_len=FAKE, B=2, D=128)
    a.update(kw)
    return lca.AppendJob(**a)


def decode_append(L, jobs, n=None):
    arr = (lca.AppendJob * max(1, len(jobs)))(*jobs)
    return L.lca_decode_append(arr, len(jobs) if n is None else n, None)


def test_window_attend_validation(L):
    a = dict(q=FAKE, q_dt=lca.BF16, win=FAKE, win_dt=lca.BF16, W_buf=256, win_begin=FAKE, win_len=FAKE, sink=FAKE,
             scale=0.088, B=2, Tq=1, Hq=64, D=128, out=FAKE, out_dt=lca.BF16, lse=None, ws=FAKE, ws_bytes=1 << 30,
             stream=None)

    def call(**kw):
        b = dict(a)
        b.update(kw)
        return L.lca_window_attend(*b.values())
    assert call(B=0) == 0
    assert call(win=None) == 1
    assert b"win must be" in L.lca_last_error()
    assert call(Hq=48) == 2
    assert call(D=64) == 2
    assert call(q_dt=lca.FP8E4M3) == 2
    need = L.lca_attend_ws(2, 1, 64, 128, 0, 256)
    if need > 0:
        assert call(ws=None) == 4


def test_decode_append_validation(L):
    assert decode_append(L, [append_job(B=0)]) == 0                        # nothing to launch
    assert decode_append(L, [append_job(B=0, x_new=None, ring=None, len=None)]) == 0
    assert decode_append(L, []) == 1
    assert decode_append(L, [append_job()] * 9) == 1
    assert L.lca_decode_append(None, 1, None) == 1
    assert decode_append(L, [append_job(x_new=None)]) == 1
    assert b"x_new" in L.lca_last_error()
    assert decode_append(L, [append_job(B=0), append_job(ring=FAKE + 2)]) == 1
    assert b"append job 1" in L.lca_last_error()
    assert decode_append(L, [append_job(len=None)]) == 1
    assert decode_append(L, [append_job(R=127)]) == 1                       # R < W
    assert decode_append(L, [append_job(m=128, W=0, R=64)]) == 1            # R < m
    assert decode_append(L, [append_job(gring=None)]) == 1                  # gate without its ring
    assert decode_append(L, [append_job(win_len=None)]) == 1
    assert decode_append(L, [append_job(m=-1)]) == 1
    assert decode_append(L, [append_job(D=96)]) == 2
    assert decode_append(L, [append_job(x_dt=lca.FP8E4M3)]) == 2


def test_decode_loop_step_validation(L):
    def call(apps, cjobs, ij=None, ajobs=()):
        pa = (lca.AppendJob * max(1, len(apps)))(*apps)
        ca = (lca.CompressJob * max(1, len(cjobs)))(*cjobs)
        aa = (lca.AttendJob * max(1, len(ajobs)))(*ajobs)
        return L.lca_decode_loop_step(pa, len(apps), ca, len(cjobs), None if ij is None else ctypes.byref(ij), aa,
                                      len(ajobs), None)
    RING, TOK0, NBLK, ROW0 = FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5
    app = lambda **kw: append_job(ring=RING, x_tok0=TOK0, nblk=NBLK, dst_row0=ROW0, R=128, m=4, **kw)
    cj = lambda **kw: batch_job(**{**dict(x=RING, x_tok0=TOK0, nblk=NBLK, dst_row0=ROW0, x_rows=256, m=4), **kw})
    # nothing to launch (every job has B = 0): accepted without a GPU
    assert call([app(B=0)], [cj(B=0)]) == 0
    assert call([], []) == 0
    assert call([app(B=0)], []) == 0
    # pairing rules
    assert call([app()], [cj(nblk=FAKE * 6)]) == 1
    assert b"x_tok0 / nblk / dst_row0" in L.lca_last_error()
    assert call([app()], [cj(nblk_max=2)]) == 1
    assert call([app()], [cj(x_rows=512)]) == 1
    assert call([app()], [cj(m=128)]) == 1
    assert call([app()], [cj(B=1)]) == 1
    assert call([app()], [cj(overlap=2)]) == 1                         # overlap differs
    assert call([app()], [cj(), cj()]) == 1
    assert b"read the ring of append job 0" in L.lca_last_error()
    # the parts are validated as their own calls
    assert call([app(D=96)], []) == 2
    assert call([app()] * 9, []) == 1
    assert call([app(B=0)], [cj(B=0)], index_job(k=0)) == 1
    assert b"index job" in L.lca_last_error()


def test_compress_variant_validation(L):
    def batch(**kw):
        arr = (lca.CompressJob * 1)(batch_job(**kw))
        return L.lca_compress_batch(arr, 1, None)
    assert batch(gate_pc=2) == 1
    assert batch(overlap=5) == 1                          # overlap > m
    assert batch(overlap=-1) == 1
    assert batch(m=1024, overlap=1, x_rows=4096) == 1     # m + overlap > 1024
    assert batch(nblk_max=64, x_rows=256, overlap=1, dst_rows=64) == 1   # span of the last block
    assert batch(B=0, gate_pc=1, overlap=4) == 0
    assert decode_append(L, [append_job(overlap=5)]) == 1
    assert decode_append(L, [append_job(m=128, W=0, R=128, overlap=1)]) == 1        # R < m + overlap
    assert decode_append(L, [append_job(B=0, m=128, W=0, R=256, overlap=128)]) == 0


def test_attend_separate_v_validation(L):
    a = dict(sparse=1, q=FAKE, q_dt=lca.BF16, k=FAKE, v=FAKE, kv_dt=lca.FP8E4M3, k_scale=FAKE, v_scale=FAKE,
             N_cap=1024, idx=FAKE, kk=64, n_elig=None, win_k=FAKE, win_v=FAKE, win_dt=lca.BF16, W_buf=256,
             win_begin=FAKE, win_len=FAKE, sink=FAKE, scale=0.088, B=2, Tq=1, Hq=64, D=128, out=FAKE,
             out_dt=lca.BF16, lse=None, ws=FAKE, ws_bytes=1 << 30, stream=None)

    def call(**kw):
        b = dict(a)
        b.update(kw)
        return L.lca_attend_separate_v(*b.values())
    assert call(B=0) == 0
    assert call(v=None) == 1
    assert b"v must be" in L.lca_last_error()
    assert call(win_v=None) == 1
    assert call(v_scale=None) == 1
    assert call(kv_dt=lca.BF16, k_scale=None) == 1          # v_scale given for bf16
    assert call(sparse=2) == 1
    assert call(idx=None) == 1
    assert call(sparse=0, idx=None, kk=0) == 1              # dense needs n_elig
    assert call(Hq=48) == 2
