"""lca_decode_step_noalloc, the decode step for callers that cannot allocate
device memory: every workspace comes from the library's per-GPU scratch.  Two
calls in a row through the C ABI -- a step at 40000 cache rows and top-512,
then a smaller one (12000 rows, top-256) -- each give the bytes of
lca_decode_step with caller workspaces on the same inputs (index sets,
selected entries' outputs, both attentions and the cache rows the step
writes).  Inputs are seeded N(0, 1) (the decode-step test's workload)."""
import ctypes

import pytest
import torch

import long_context_attention_13_amd as lca
from test_gpu_step import Step

pytestmark = pytest.mark.gpu


def noalloc(st):
    ca = (lca.CompressJob * len(st.cjobs))(*st.cjobs)
    aa = (lca.AttendJob * len(st.ajobs))(*st.ajobs)
    lca._check(lca.load().lca_decode_step_noalloc(ca, len(st.cjobs), ctypes.byref(st.ijob), aa, len(st.ajobs),
                                                  lca._stream(None)))


def test_noalloc_step_equals_decode_step():
    for seed, N, N2, k in [(951, 40000, 320, 512), (952, 12000, 100, 256)]:
        print(f"decode_step_noalloc: N={N} N2={N2} k={k}", flush=True)
        st = Step(seed, N=N, N2=N2, k=k)
        st.step()
        torch.cuda.synchronize()
        ref = st.outputs()
        st.clobber()
        noalloc(st)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(st.outputs(), ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"N={N}: output {i}"
