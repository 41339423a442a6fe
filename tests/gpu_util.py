"""Helpers for the GPU parity tests: host<->device transfer of the storage
types and the comparison rule for floating-point outputs."""
import numpy as np
import torch

import long_context_attention_13_amd as lca


def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    lca.load()          # fails loudly if the HIP library is not built
    return torch.device("cuda:0")


def to_dev(a, bf16=False):
    """numpy -> device tensor.  uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
    t = torch.from_numpy(a).to(dev())
    return t.to(torch.bfloat16) if bf16 else t


def to_host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_rows_close(got, ref, rtol, what=""):
    """|got - ref| <= rtol * (|ref| + max |ref| over the row), row = last dim.

    The comparison rule for attention outputs and pooled rows: an element is
    held to rtol of its own magnitude plus rtol of the largest magnitude in its
    row (one head's output vector, one pooled entry), so elements near zero in
    a row of ordinary size are not held to a vanishing bound."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rowmax = np.abs(ref).max(axis=-1, keepdims=True) if ref.size else ref
    tol = rtol * (np.abs(ref) + rowmax)
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside rtol {rtol}; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} tol {tol[i]!r}")


def assert_lse_close(got, ref, rtol, what=""):
    """Log-sum-exp rows: |got - ref| <= rtol * max(|ref|, 1), element by element.

    The tolerance is relative to the LSE itself (no row floor: each element is
    its own row); below |lse| = 1 it is relative to the softmax normaliser
    Z = exp(lse) instead, since |d lse| = |dZ| / Z, so an LSE near zero is not
    held to a vanishing absolute bound."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    tol = rtol * np.maximum(np.abs(ref), 1.0)
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside rtol {rtol}; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} tol {tol[i]!r}")


def empty_ws(nbytes):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=dev())
