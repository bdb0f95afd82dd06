"""Seeded synthetic jagged batches.

The pages (Meta's GEM training post, "Challenge 1": jagged inputs and the
three asymmetric attention shapes) describe user-history sequences of wildly
varying length, long-Q/short-KV cross-attention and short-Q/long-KV pooling
attention, but publish no shapes.  The five workloads below stand in for
those production shapes; their recipe is fixed here once so that every
consumer (oracle, GPU tests, benchmark) sees bit-identical inputs.

Draw order per case: lengths, then Q, K, V, then bias, then dO.  Values are
drawn as float32 standard normals with numpy's PCG64 and rounded to the
storage dtype with torch's round-to-nearest-even cast.

Nothing here computes offsets, scores or quantised codes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

MODES = ("softmax", "silu", "gelu")
BIAS_KINDS = ("none", "relpos", "dense")
DTYPES = ("f32", "bf16", "mxfp8")


def _lognormal_lengths(rng: np.random.Generator, n: int, median: float, lo: int, hi: int,
                       sigma: float = 1.0) -> np.ndarray:
    """Log-normal lengths: round(exp(N(ln median, sigma))) clipped to [lo, hi]."""
    x = np.exp(rng.normal(math.log(median), sigma, size=n))
    return np.clip(np.floor(x + 0.5), lo, hi).astype(np.int32)


# name -> description of one workload (the five jagged-attention workloads)
WORKLOADS = {
    1: dict(name="tiny-selfattn-softmax-f32", batch=4, heads=2, head_dim=64, dtype="f32",
            mode="softmax", causal=False, bias_kind="none", forward_only=False),
    2: dict(name="causal-selfattn-relpos-bf16", batch=64, heads=4, head_dim=128, dtype="bf16",
            mode="softmax", causal=True, bias_kind="relpos", forward_only=False),
    3: dict(name="gdpa-silu-crossattn-bf16", batch=256, heads=8, head_dim=128, dtype="bf16",
            mode="silu", causal=False, bias_kind="none", forward_only=False),
    4: dict(name="gdpa-gelu-shortkv-densebias-bf16", batch=2048, heads=4, head_dim=64,
            dtype="bf16", mode="gelu", causal=False, bias_kind="dense", forward_only=False),
    5: dict(name="mxfp8-causal-selfattn-fwd", batch=256, heads=4, head_dim=128, dtype="mxfp8",
            mode="softmax", causal=True, bias_kind="none", forward_only=True),
}


def lengths_for(cfg: int, rng: np.random.Generator, batch: Optional[int] = None):
    """Per-sample (q_len, kv_len) for workload ``cfg``; ``batch`` overrides B."""
    c = WORKLOADS[cfg]
    B = c["batch"] if batch is None else batch
    if cfg == 1:
        q = rng.integers(1, 129, size=B).astype(np.int32)
        if B > 1:
            q[1] = 0          # one interior sample forced empty
        return q, q.copy()
    if cfg == 2:
        q = _lognormal_lengths(rng, B, 512, 16, 4096)
        return q, q.copy()
    if cfg == 3:
        q = rng.integers(16, 65, size=B).astype(np.int32)
        kv = _lognormal_lengths(rng, B, 256, 32, 2048)
        return q, kv
    if cfg == 4:
        q = np.full(B, 256, dtype=np.int32)
        kv = rng.integers(8, 65, size=B).astype(np.int32)
        return q, kv
    if cfg == 5:
        q = _lognormal_lengths(rng, B, 512, 16, 8192)
        return q, q.copy()
    raise ValueError(f"unknown workload {cfg}")


@dataclass
class Case:
    """One jagged batch.  Tensors live on the CPU in their storage dtype."""
    name: str
    q_lens: np.ndarray
    kv_lens: np.ndarray
    heads: int
    head_dim: int
    dtype: str
    mode: str
    causal: bool
    bias_kind: str
    num_buckets: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    bias: Optional[torch.Tensor]
    dout: Optional[torch.Tensor]
    forward_only: bool = False
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def total_kv(self) -> int:
        return int(self.kv_lens.sum())


def _normals(rng, shape, dtype: torch.dtype) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def custom_case(q_lens, kv_lens, heads: int, head_dim: int, *, dtype: str = "bf16",
                mode: str = "softmax", causal: bool = False, bias_kind: str = "none",
                num_buckets: int = 64, seed: int = 0, with_dout: bool = True,
                bias_std: float = 0.1, name: str = "custom",
                rng: Optional[np.random.Generator] = None) -> Case:
    """Builds a batch with the given per-sample lengths (drawn after the lengths)."""
    assert mode in MODES and bias_kind in BIAS_KINDS and dtype in DTYPES
    q_lens = np.asarray(q_lens, dtype=np.int32)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    assert q_lens.shape == kv_lens.shape
    if rng is None:
        rng = np.random.default_rng(seed)
    store = torch.float32 if dtype == "f32" else torch.bfloat16
    Tq, Tkv = int(q_lens.sum()), int(kv_lens.sum())
    q = _normals(rng, (Tq, heads, head_dim), store)
    k = _normals(rng, (Tkv, heads, head_dim), store)
    v = _normals(rng, (Tkv, heads, head_dim), store)
    bias = None
    if bias_kind == "relpos":
        bias = (torch.from_numpy(rng.standard_normal(size=(heads, num_buckets), dtype=np.float32))
                * bias_std).to(torch.float32)
    elif bias_kind == "dense":
        n_elem = int(heads * np.sum(q_lens.astype(np.int64) * kv_lens.astype(np.int64)))
        bias = (torch.from_numpy(rng.standard_normal(size=n_elem, dtype=np.float32)) * bias_std
                ).to(store)
    dout = _normals(rng, (Tq, heads, head_dim), store) if with_dout else None
    return Case(name=name, q_lens=q_lens, kv_lens=kv_lens, heads=heads, head_dim=head_dim,
                dtype=dtype, mode=mode, causal=causal, bias_kind=bias_kind,
                num_buckets=num_buckets, q=q, k=k, v=v, bias=bias, dout=dout,
                forward_only=not with_dout, seed=seed)


def make_case(cfg: int, seed: Optional[int] = None, batch: Optional[int] = None,
              with_dout: Optional[bool] = None) -> Case:
    """Workload ``cfg`` (1..5) drawn with ``seed`` (default: the workload number).  with_dout
    overrides whether dO is drawn (last, so Q, K, V and the bias do not change)."""
    c = WORKLOADS[cfg]
    seed = cfg if seed is None else seed
    rng = np.random.default_rng(seed)
    q_lens, kv_lens = lengths_for(cfg, rng, batch)
    want_dout = (not c["forward_only"]) if with_dout is None else bool(with_dout)
    case = custom_case(q_lens, kv_lens, c["heads"], c["head_dim"], dtype=c["dtype"],
                       mode=c["mode"], causal=c["causal"], bias_kind=c["bias_kind"],
                       seed=seed, with_dout=want_dout, name=c["name"], rng=rng)
    case.extra["config"] = cfg
    return case
