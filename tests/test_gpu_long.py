"""A long sample: one causal sequence of 32,768 tokens (eight times the workloads' cap), relative-
position bias, softmax.  Causal rows depend only on the keys up to themselves, so the first rows
of the long sample must equal the oracle on that prefix taken as a sample of its own; the last
row, which sees every key, is checked against a direct fp64 evaluation of that one row."""
import math

import numpy as np
import pytest
import torch

import oracle
from jfa_synth import custom_case
from tests.gpu_helpers import compare, say

pytestmark = pytest.mark.gpu

N, PREFIX, H, D = 32768, 1536, 2, 128


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


def test_long_causal_sample_forward():
    import jagged_attention_amd as jfa
    case = custom_case([N], [N], H, D, dtype="bf16", mode="softmax", causal=True,
                       bias_kind="relpos", seed=61, with_dout=False)
    say(f"[long] n={N}")
    dev = torch.device("cuda:0")
    off = torch.tensor([0, N], dtype=torch.int32, device=dev)
    q, k, v = (t.to(dev) for t in (case.q, case.k, case.v))
    bias = case.bias.to(dev)
    o, lse = jfa.forward(q, k, v, off, off, causal=True, bias=bias, bias_kind="relpos")
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    # the prefix as a sample of its own (oracle)
    pq, pk, pv = case.q[:PREFIX], case.k[:PREFIX], case.v[:PREFIX]
    o_ref, lse_ref = oracle.forward(pq, pk, pv, [PREFIX], [PREFIX], causal=True, bias=case.bias,
                                    bias_kind="relpos")
    compare("O[prefix]", o[:PREFIX], o_ref, "bf16")
    assert np.max(np.abs(lse[:, :PREFIX].cpu().double().numpy() - lse_ref)) < 1e-3
    # the last row over all N keys, in fp64
    i = N - 1
    for h in range(H):
        qi = case.q[i, h].double()
        kk = case.k[:, h].double()
        dist = torch.arange(N - 1, -1, -1)          # i - j for j = 0 .. N-1
        buckets = torch.tensor([oracle.relpos_bucket(int(x)) for x in dist.tolist()])
        srow = (kk @ qi) / math.sqrt(D) + case.bias[h].double()[buckets]
        p = torch.softmax(srow, dim=0)
        want = p @ case.v[:, h].double()
        got = o[i, h].float().cpu().double()
        err = (got - want).abs().max().item()
        assert err < 2e-2, (h, err)
        assert abs(lse[h, i].item() - torch.logsumexp(srow, 0).item()) < 1e-3
