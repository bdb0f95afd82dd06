"""Independent fp64 references used to pin the oracle (tests only).

These are written against torch's own routines (scaled_dot_product_attention,
autograd, silu/gelu) and dense padded tensors, never against the oracle's
source, so a mistake in the oracle shows up as a disagreement.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def per_sample_views(x: torch.Tensor, lens):
    off = 0
    out = []
    for n in lens:
        out.append(x[off:off + int(n)])
        off += int(n)
    return out


def bias_matrix(bias, bias_kind, h, n, m, H, b_index, q_lens, kv_lens, bucket_fn, num_buckets=64):
    """Dense [n, m] bias of sample b_index, head h (fp64)."""
    if bias_kind == "none":
        return torch.zeros(n, m, dtype=torch.float64)
    if bias_kind == "relpos":
        table = torch.as_tensor(bias, dtype=torch.float64)
        out = torch.zeros(n, m, dtype=torch.float64)
        for i in range(n):
            for j in range(m):
                out[i, j] = table[h, bucket_fn(i + (m - n) - j, num_buckets)]
        return out
    # dense jagged: sample blocks laid out one after another, each [H, n, m]
    start = 0
    for bb in range(b_index):
        start += H * int(q_lens[bb]) * int(kv_lens[bb])
    blk = torch.as_tensor(bias, dtype=torch.float64)[start:start + H * n * m].reshape(H, n, m)
    return blk[h].clone()


def visible_mask(n, m, causal, window=0):
    """[n, m] visibility: causal bottom-right (j <= i + m - n); a sliding window keeps keys with
    |i + m - n - j| < window (a band of the dense matrix)."""
    i = torch.arange(n)[:, None]
    j = torch.arange(m)[None, :]
    vis = torch.ones(n, m, dtype=torch.bool)
    if causal:
        vis = vis & (j <= i + (m - n))
    if window:
        vis = vis & ((i + (m - n) - j).abs() < window)
    return vis


def sdpa_sample(q, k, v, bmat, vis, scale):
    """Softmax attention of one (sample, head) via torch's SDPA (math path, fp64).

    q [n,d], k/v [m,d]; returns (o [n,d], lse [n]).  Rows with no visible key
    come back as NaN from torch; the caller handles them."""
    mask = bmat.clone()
    mask[~vis] = -math.inf
    o = F.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None],
                                       attn_mask=mask[None, None], scale=scale)[0, 0]
    s = scale * (q @ k.T) + mask
    lse = torch.logsumexp(s, dim=1)
    return o, lse


def gdpa_sample(q, k, v, bmat, vis, scale, mode, normalize=True):
    """GDPA of one (sample, head) with torch's activations (fp64)."""
    s = scale * (q @ k.T) + bmat
    a = F.silu(s) if mode == "silu" else F.gelu(s, approximate="none")
    a = torch.where(vis, a, torch.zeros_like(a))
    m = k.shape[0]
    w = (1.0 / m) if (normalize and m > 0) else 1.0
    return w * (a @ v)


def torch_reference(case_q, case_k, case_v, q_lens, kv_lens, mode, causal, bias, bias_kind,
                    bucket_fn, scale=None, dout=None, num_buckets=64, window=0):
    """Per-sample fp64 torch reference, with autograd gradients when dout is given.

    Returns dict(o, lse, dq, dk, dv) as fp64 numpy arrays (lse NaN for GDPA)."""
    q = torch.as_tensor(np.asarray(case_q, dtype=np.float64)).clone()
    k = torch.as_tensor(np.asarray(case_k, dtype=np.float64)).clone()
    v = torch.as_tensor(np.asarray(case_v, dtype=np.float64)).clone()
    Tq, H, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    want_grad = dout is not None
    if want_grad:
        q.requires_grad_(True)
        k.requires_grad_(True)
        v.requires_grad_(True)
    o_all = torch.zeros(Tq, H, d, dtype=torch.float64)
    lse_all = torch.full((H, Tq), float("nan"), dtype=torch.float64)
    outs = []
    qo = 0
    ko = 0
    for b, (n, m) in enumerate(zip(q_lens, kv_lens)):
        n, m = int(n), int(m)
        for h in range(H):
            if n == 0:
                continue
            qs, ks, vs = q[qo:qo + n, h], k[ko:ko + m, h], v[ko:ko + m, h]
            vis = visible_mask(n, m, causal, window)
            bmat = bias_matrix(bias, bias_kind, h, n, m, H, b, q_lens, kv_lens, bucket_fn,
                               num_buckets)
            if mode == "softmax":
                if m == 0:
                    o = torch.zeros(n, d, dtype=torch.float64)
                    lse = torch.full((n,), -math.inf, dtype=torch.float64)
                else:
                    o, lse = sdpa_sample(qs, ks, vs, bmat, vis, scale)
                    dead = ~vis.any(dim=1)
                    o = torch.where(dead[:, None], torch.zeros_like(o), o)
                    lse = torch.where(dead, torch.full_like(lse, -math.inf), lse)
                lse_all[h, qo:qo + n] = lse.detach()
            else:
                o = gdpa_sample(qs, ks, vs, bmat, vis, scale, mode) if m > 0 else \
                    torch.zeros(n, d, dtype=torch.float64)
            outs.append((qo, n, h, o))
        qo += n
        ko += m
    for (qo_, n, h, o) in outs:
        o_all[qo_:qo_ + n, h] = o.detach()
    res = dict(o=o_all.numpy(), lse=lse_all.numpy())
    if want_grad:
        loss = torch.zeros((), dtype=torch.float64)
        dO = torch.as_tensor(np.asarray(dout, dtype=np.float64))
        for (qo_, n, h, o) in outs:
            loss = loss + (o * dO[qo_:qo_ + n, h]).sum()
        if loss.requires_grad:
            gq, gk, gv = torch.autograd.grad(loss, (q, k, v), allow_unused=True)
        else:
            gq = gk = gv = None
        res["dq"] = (gq if gq is not None else torch.zeros_like(q)).detach().numpy()
        res["dk"] = (gk if gk is not None else torch.zeros_like(k)).detach().numpy()
        res["dv"] = (gv if gv is not None else torch.zeros_like(v)).detach().numpy()
    return res


def rel_l2(x, y) -> float:
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    den = np.linalg.norm(y)
    num = np.linalg.norm(x - y)
    return float(num / den) if den > 0 else float(num)


def max_abs(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(x - y))) if x.size else 0.0
