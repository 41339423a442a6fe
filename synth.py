"""Seeded synthetic inputs for the CSA/HCA hot path.

This module only draws random numbers: it holds none of the method's
arithmetic (no pooling, no quantisation, no scoring).  Both the GPU path's
tests and the float64 oracle consume what it returns, so it is the single
shared piece between them.

Workloads (shapes and distributions of the five configurations the hot path is
measured on; the pages give no data set, only context lengths, so everything
is Gaussian or uniform noise with these shapes):

  small_csa_decode   1 sequence, 4096 tokens, fp32, m=4 -> 1024 entries,
                     16 query heads, indexer 4 heads x 64, top-64, window 128
  hca_decode_bf16    8 sequences x 65536 tokens, bf16, m'=128 -> 512 entries,
                     64 query heads, window 128
  csa_decode_fp8     16 sequences x 131072 tokens: 32768 FP8 entries,
                     MXFP4 indexer keys (8 heads x 128), top-512, window 128
  layer_pair_1m      4 sequences, capacity 2^20 tokens, lengths uniform in
                     [0.9 * 2^20, 2^20]: 262144 FP8 CSA entries + MXFP4 keys,
                     top-1024; 8192 FP8 HCA entries; window 128; 64 heads
  prefill_chunk      8192 new bf16 tokens after a 262144-token cache
  v4_pro schedule    the attention layers of the 61-layer model and its MTP
                     block (v4_pro_layer_kinds), each layer with caches of the
                     layer_pair_1m shapes and its own raw-token rings

Distributions: KV, gates, queries, raw keys ~ N(0,1); positional bias ~
N(0, 0.1^2); indexer head weights ~ U(0,1); sinks ~ N(0,1); the small fp32
configuration scales Q by 1/sqrt(128) and uses softmax scale 1, the others use
softmax scale 1/sqrt(128).  numpy's PCG64 generator is seeded per workload
(1001..1005) and every array is drawn in a fixed order.
"""
from __future__ import annotations

import math

import numpy as np

SEEDS = {
    "small_csa_decode": 1001,
    "hca_decode_bf16": 1002,
    "csa_decode_fp8": 1003,
    "layer_pair_1m": 1004,
    "prefill_chunk": 1005,
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def uniform(g: np.random.Generator, shape) -> np.ndarray:
    return g.random(size=shape, dtype=np.float32)


def small_csa_decode(seed: int = SEEDS["small_csa_decode"], L: int = 4096, Hq: int = 16,
                     H_I: int = 4, d_I: int = 64, D: int = 128, W: int = 128, m: int = 4,
                     k: int = 64):
    """One sequence of raw tokens; the cache is built by pooling them."""
    g = rng(seed)
    out = dict(B=1, L=L, Hq=Hq, H_I=H_I, d_I=d_I, D=D, W=W, m=m, k=k, tau=1.0)
    out["x"] = normal(g, (1, L, D))                 # raw KV tokens
    out["gate"] = normal(g, (1, L))                 # pooling gate logits
    out["bias"] = normal(g, (m,), 0.1)              # positional bias
    out["xi"] = normal(g, (1, L, d_I))              # raw indexer keys
    out["gate_i"] = normal(g, (1, L))               # indexer pooling gate
    out["bias_i"] = normal(g, (m,), 0.1)
    out["qi"] = normal(g, (1, 1, H_I, d_I))          # indexer query
    out["w"] = uniform(g, (1, 1, H_I))               # indexer head weights
    out["sink"] = normal(g, (Hq,))
    out["q"] = (normal(g, (1, 1, Hq, D)) / np.float32(math.sqrt(128.0))).astype(np.float32)
    return out


def hca_decode_bf16(seed: int = SEEDS["hca_decode_bf16"], B: int = 8, L: int = 65536,
                    Hq: int = 64, D: int = 128, W: int = 128, m: int = 128):
    g = rng(seed)
    out = dict(B=B, L=L, Hq=Hq, D=D, W=W, m=m, tau=1.0 / math.sqrt(128.0))
    out["x"] = normal(g, (B, L, D))
    out["gate"] = normal(g, (B, L))
    out["bias"] = normal(g, (m,), 0.1)
    out["sink"] = normal(g, (Hq,))
    out["q"] = normal(g, (B, 1, Hq, D))
    return out


def csa_decode_fp8(seed: int = SEEDS["csa_decode_fp8"], B: int = 16, L: int = 131072,
                   Hq: int = 64, H_I: int = 8, d_I: int = 128, D: int = 128, W: int = 128,
                   m: int = 4, k: int = 512):
    """The compressed caches are drawn directly (values before quantisation)."""
    g = rng(seed)
    N = L // m
    out = dict(B=B, L=L, N=N, Hq=Hq, H_I=H_I, d_I=d_I, D=D, W=W, m=m, k=k,
               tau=1.0 / math.sqrt(128.0))
    out["entries"] = normal(g, (B, N, D))
    out["keys"] = normal(g, (B, N, d_I))
    out["qi"] = normal(g, (B, 1, H_I, d_I))
    out["w"] = uniform(g, (B, 1, H_I))
    out["sink"] = normal(g, (Hq,))
    out["q"] = normal(g, (B, 1, Hq, D))
    out["win"] = normal(g, (B, W, D))
    return out


def layer_pair_1m(seed: int = SEEDS["layer_pair_1m"], B: int = 4, cap: int = 1 << 20,
                  Hq: int = 64, H_I: int = 8, d_I: int = 128, D: int = 128, W: int = 128,
                  m: int = 4, m2: int = 128, k: int = 1024, draw_caches: bool = True):
    """Lengths uniform over the integers [ceil(0.9*cap), cap]."""
    g = rng(seed)
    lo = -(-9 * cap // 10)
    L = g.integers(lo, cap + 1, size=B).astype(np.int64)
    out = dict(B=B, cap=cap, L=L, N_cap=cap // m, N2_cap=cap // m2, Hq=Hq, H_I=H_I, d_I=d_I,
               D=D, W=W, m=m, m2=m2, k=k, tau=1.0 / math.sqrt(128.0))
    out["qi"] = normal(g, (B, 1, H_I, d_I))
    out["w"] = uniform(g, (B, 1, H_I))
    out["sink_csa"] = normal(g, (Hq,))
    out["sink_hca"] = normal(g, (Hq,))
    out["q_csa"] = normal(g, (B, 1, Hq, D))
    out["q_hca"] = normal(g, (B, 1, Hq, D))
    out["win_csa"] = normal(g, (B, W, D))
    out["win_hca"] = normal(g, (B, W, D))
    out["win_keys"] = normal(g, (B, W, d_I))
    out["gate_csa"] = normal(g, (B, W))
    out["gate_i"] = normal(g, (B, W))
    out["gate_hca"] = normal(g, (B, W))
    out["bias_csa"] = normal(g, (m,), 0.1)
    out["bias_i"] = normal(g, (m,), 0.1)
    out["bias_hca"] = normal(g, (m2,), 0.1)
    if draw_caches:
        out["entries"] = normal(g, (B, cap // m, D))
        out["keys"] = normal(g, (B, cap // m, d_I))
        out["hca_entries"] = normal(g, (B, cap // m2, D))
    return out


def prefill_chunk(seed: int = SEEDS["prefill_chunk"], ctx: int = 262144, T: int = 8192,
                  Hq: int = 64, H_I: int = 8, d_I: int = 128, D: int = 128, W: int = 128,
                  m: int = 4, m2: int = 128, k: int = 1024):
    """Cached compressed entries are drawn directly; the new chunk is raw."""
    g = rng(seed)
    out = dict(B=1, ctx=ctx, T=T, Hq=Hq, H_I=H_I, d_I=d_I, D=D, W=W, m=m, m2=m2, k=k,
               tau=1.0 / math.sqrt(128.0))
    out["entries_old"] = normal(g, (1, ctx // m, D))
    out["keys_old"] = normal(g, (1, ctx // m, d_I))
    out["hca_old"] = normal(g, (1, ctx // m2, D))
    out["x_prev"] = normal(g, (1, W - 1, D))        # raw tokens just before the chunk
    out["x"] = normal(g, (1, T, D))
    out["gate"] = normal(g, (1, T))
    out["bias"] = normal(g, (m,), 0.1)
    out["xi"] = normal(g, (1, T, d_I))
    out["gate_i"] = normal(g, (1, T))
    out["bias_i"] = normal(g, (m,), 0.1)
    out["gate2"] = normal(g, (1, T))
    out["bias2"] = normal(g, (m2,), 0.1)
    out["qi"] = normal(g, (1, T, H_I, d_I))
    out["w"] = uniform(g, (1, T, H_I))
    out["sink_csa"] = normal(g, (Hq,))
    out["sink_hca"] = normal(g, (Hq,))
    out["q"] = normal(g, (1, T, Hq, D))
    return out


def v4_pro_layer_kinds(n_layers: int = 61) -> list:
    """Attention kind of every layer of the 61-layer V4-Pro model, then its MTP
    block: layers 0 and 1 "hca", layers 2 .. n_layers-1 alternating "csa" and
    "hca" starting with "csa", and "window" (sliding-window attention only)
    for the MTP block.  A configuration list, not arithmetic."""
    return ["hca", "hca"] + ["csa" if (l - 2) % 2 == 0 else "hca" for l in range(2, n_layers)] + ["window"]
