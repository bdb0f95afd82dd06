"""Robustness of the HIP path beyond element-wise parity:

- guard bands: every output (O, LSE, dQ, dK, dV, a dense dβ) and the workspace sit inside a
  larger buffer filled with a sentinel; after the call the bands are unchanged, so no kernel
  stores past a tensor's ends, and the outputs equal a plain call's bit for bit;
- batch order: the samples of a batch in another order give each sample the same results bit for
  bit (the longest-first lists and the per-XCD ticket order then differ completely; each
  sample's sums run in a fixed order whatever workgroup takes its tiles);
- a long sample in the backward: a causal sequence of 8192 tokens (twice the workloads' cap)
  whose dO is zero outside its last 512 rows, so that every gradient depends on those rows only
  and equals the oracle on the sample made of those 512 queries and all 8192 keys (causal
  alignment puts query i of that sample at position 7680 + i).
"""
import numpy as np
import pytest
import torch

import oracle
from jfa_synth import custom_case, make_case
from tests.gpu_helpers import compare, device_case, say

pytestmark = pytest.mark.gpu

GUARD = 4096        # elements of sentinel on each side (a multiple of 16 bytes for every dtype)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


def guarded(shape, dtype, fill):
    """(full buffer, view of the middle with `shape`); the bands hold `fill`."""
    n = int(np.prod(shape))
    buf = torch.full((GUARD + n + GUARD,), fill, dtype=dtype, device="cuda:0")
    return buf, buf[GUARD:GUARD + n].view(shape)


def bands_intact(buf, fill):
    want = torch.full((GUARD,), fill, dtype=buf.dtype, device=buf.device)
    return torch.equal(buf[:GUARD], want) and torch.equal(buf[-GUARD:], want)


def run_guarded(case, dbias=False):
    """Forward and backward with every output and both workspaces inside guard bands."""
    import jagged_attention_amd as jfa
    dc = device_case(case)
    p = jfa.make_problem(case.batch, case.heads, case.head_dim, case.total_q, case.total_kv,
                         mode=case.mode, causal=case.causal, bias_kind=case.bias_kind,
                         num_buckets=case.num_buckets)
    fills = {torch.bfloat16: -7.0, torch.float32: -7.0, torch.uint8: 0xA5}
    bufs = []

    def out(shape, dtype):
        b, v = guarded(shape, dtype, fills[dtype])
        bufs.append(b)
        return v

    o = out(tuple(dc["q"].shape), torch.bfloat16)
    lse = out((case.heads, case.total_q), torch.float32) if case.mode == "softmax" else None
    nf = jfa.jfa_workspace_bytes(p, False)
    wsf = out((nf,), torch.uint8)          # GUARD bytes past a 512-byte aligned allocation
    jfa.jfa_forward(p, dc["q"], dc["k"], dc["v"], None, None, None, dc["qo"], dc["ko"],
                    dc["bias"], o, lse, wsf, nf)
    dq = out(tuple(dc["q"].shape), torch.bfloat16)
    dk = out(tuple(dc["k"].shape), torch.bfloat16)
    dv = out(tuple(dc["v"].shape), torch.bfloat16)
    nb = jfa.jfa_workspace_bytes(p, 2 if dbias else 1)
    wsb = out((nb,), torch.uint8)
    db = None
    if dbias:
        db = out(tuple(dc["bias"].shape), dc["bias"].dtype)   # fp32 table or bf16 dense
        jfa.jfa_backward_dbias(p, dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"],
                               dc["ko"], dc["bias"], dq, dk, dv, db, wsb, nb)
    else:
        jfa.jfa_backward(p, dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"], dc["ko"],
                         dc["bias"], dq, dk, dv, wsb, nb)
    torch.cuda.synchronize()
    for b in bufs:
        assert bands_intact(b, fills[b.dtype]), "a kernel wrote outside its buffer"
    return dc, [t for t in (o, lse, dq, dk, dv, db) if t is not None]


@pytest.mark.parametrize("cfg,batch,dbias", [(2, 12, False), (3, 40, False), (4, 48, True),
                                              (2, 12, True)])
def test_outputs_stay_inside_their_buffers(cfg, batch, dbias):
    import jagged_attention_amd as jfa
    case = make_case(cfg, batch=batch, with_dout=True)
    say(f"[guard] cfg={cfg} B={batch} dbias={dbias}")
    dc, got = run_guarded(case, dbias)
    # the same call on plain tensors: identical bits
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], mode=case.mode,
                         causal=case.causal, bias=dc["bias"], bias_kind=case.bias_kind,
                         num_buckets=case.num_buckets)
    if dbias:
        dq, dk, dv, db = jfa.backward_dbias(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"],
                                            dc["qo"], dc["ko"], dc["bias"], mode=case.mode,
                                            causal=case.causal, bias_kind=case.bias_kind,
                                            num_buckets=case.num_buckets)
        want = [o, lse, dq, dk, dv, db]
    else:
        dq, dk, dv = jfa.backward(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"],
                                  dc["ko"], mode=case.mode, causal=case.causal, bias=dc["bias"],
                                  bias_kind=case.bias_kind, num_buckets=case.num_buckets)
        want = [o, lse, dq, dk, dv]
    want = [t for t in want if t is not None]
    torch.cuda.synchronize()
    assert len(got) == len(want)
    for g, w in zip(got, want):
        assert torch.equal(g, w)


def permuted_case(case, perm):
    """The same samples in the order `perm` (the dense bias's per-sample blocks move along)."""
    qo = oracle.offsets(case.q_lens)
    ko = oracle.offsets(case.kv_lens)
    cat = lambda x, off: torch.cat([x[off[b]:off[b + 1]] for b in perm])
    c = custom_case(case.q_lens[perm], case.kv_lens[perm], case.heads, case.head_dim,
                    dtype=case.dtype, mode=case.mode, causal=case.causal,
                    bias_kind=case.bias_kind, num_buckets=case.num_buckets)
    c.q, c.k, c.v = cat(case.q, qo), cat(case.k, ko), cat(case.v, ko)
    c.dout = cat(case.dout, qo)
    if case.bias_kind == "dense":
        bo = oracle.bias_offsets(case.q_lens, case.kv_lens) * case.heads
        c.bias = torch.cat([case.bias[bo[b]:bo[b + 1]] for b in perm])
    else:
        c.bias = case.bias
    return c


def gpu_fwd_bwd(case, split_slots=0):
    import jagged_attention_amd as jfa
    dc = device_case(case)
    kw = dict(mode=case.mode, causal=case.causal, bias=dc["bias"], bias_kind=case.bias_kind,
              num_buckets=case.num_buckets)
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], split_slots=split_slots,
                         **kw)
    dq, dk, dv = jfa.backward(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"], dc["ko"],
                              **kw)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o, dq, dk, dv)], (None if lse is None else lse.cpu())


@pytest.mark.parametrize("cfg,batch,split", [(2, 16, 0), (2, 16, 4), (3, 64, 0), (4, 96, 0)])
def test_batch_order_invariance(cfg, batch, split):
    case = make_case(cfg, batch=batch, with_dout=True)
    perm = np.random.default_rng(7).permutation(batch)
    say(f"[order] cfg={cfg} B={batch} split_slots={split}")
    (o, dq, dk, dv), lse = gpu_fwd_bwd(case, split)
    (po, pdq, pdk, pdv), plse = gpu_fwd_bwd(permuted_case(case, perm), split)
    qo, ko = oracle.offsets(case.q_lens), oracle.offsets(case.kv_lens)
    pqo = oracle.offsets(case.q_lens[perm])
    pko = oracle.offsets(case.kv_lens[perm])
    for i, b in enumerate(perm):
        q0, q1, k0, k1 = qo[b], qo[b + 1], ko[b], ko[b + 1]
        p0, p1, r0, r1 = pqo[i], pqo[i + 1], pko[i], pko[i + 1]
        assert torch.equal(o[q0:q1], po[p0:p1]), ("O", b)
        assert torch.equal(dq[q0:q1], pdq[p0:p1]), ("dQ", b)
        assert torch.equal(dk[k0:k1], pdk[r0:r1]), ("dK", b)
        assert torch.equal(dv[k0:k1], pdv[r0:r1]), ("dV", b)
        if lse is not None:
            assert torch.equal(lse[:, q0:q1], plse[:, p0:p1]), ("LSE", b)


def test_long_causal_sample_backward():
    import jagged_attention_amd as jfa
    N, A, H, D = 8192, 7680, 2, 128
    case = custom_case([N], [N], H, D, dtype="bf16", mode="softmax", causal=True,
                       bias_kind="relpos", seed=62)
    case.dout[:A] = 0
    say(f"[long-bwd] n={N} dO rows {A}..{N}")
    dc = device_case(case)
    kw = dict(causal=True, bias=dc["bias"], bias_kind="relpos")
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], **kw)
    dq, dk, dv = jfa.backward(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"], dc["ko"],
                              **kw)
    torch.cuda.synchronize()
    # rows without dO have no gradient at all
    assert not dq[:A].any()
    # the last N - A queries over all N keys, as a sample of its own
    rq, rk, rv = oracle.backward(case.q[A:], case.k, case.v, case.dout[A:], [N - A], [N],
                                 causal=True, bias=case.bias, bias_kind="relpos")
    compare("dQ[long rows]", dq[A:], rq, "bf16")
    compare("dK[long]", dk, rk, "bf16")
    compare("dV[long]", dv, rv, "bf16")
