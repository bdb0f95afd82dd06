"""The forward entry point that allocates nothing (jfa_forward_noalloc), through the C ABI: its
workspace is the library's fixed per-GPU array, and its results equal jfa_forward's bit for bit
(same kernels, same tile lists) on two calls in a row, the second smaller than the first (the
array still holds the first call's contents).  Also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from jfa_synth import custom_case
from tests.gpu_helpers import compare, device_case, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode,causal,bias_kind", [("softmax", True, "relpos"),
                                                    ("gelu", False, "dense")])
def test_noalloc_forward_matches_forward(mode, causal, bias_kind):
    import jagged_attention_amd as jfa
    jfa.load()
    oracle.build()
    for lens in ([3000, 700, 0, 129, 1500], [300, 17]):
        kl = lens if causal else [max(1, x // 3) for x in lens]
        case = custom_case(lens, kl, 4, 128, dtype="bf16", mode=mode, causal=causal,
                           bias_kind=bias_kind, seed=191 + len(lens))
        say(f"[noalloc] mode={mode} q_lens={lens}")
        dc = device_case(case)
        kw = dict(mode=mode, causal=causal, bias=dc["bias"], bias_kind=bias_kind,
                  num_buckets=case.num_buckets)
        o_ref, lse_ref = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], **kw)
        p = jfa.make_problem(case.batch, case.heads, case.head_dim, case.total_q,
                             case.total_kv, mode=mode, causal=causal, bias_kind=bias_kind,
                             num_buckets=case.num_buckets)
        assert 0 < jfa.jfa_workspace_bytes(p, 0) <= jfa._lib.NOALLOC_SCRATCH_BYTES
        o = torch.full_like(o_ref, float("nan"))
        lse = None if lse_ref is None else torch.full_like(lse_ref, float("nan"))
        jfa.jfa_forward_noalloc(p, dc["q"], dc["k"], dc["v"], None, None, None, dc["qo"],
                                dc["ko"], dc["bias"], o, lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        if lse is not None:
            assert torch.equal(lse, lse_ref)
        want, _ = oracle.case_forward(case)
        compare("O", o, want, "bf16")


def test_noalloc_rejects_oversized_problem():
    """A problem whose workspace exceeds the fixed array is refused before anything runs."""
    import jagged_attention_amd as jfa
    p = jfa.make_problem(4, 16, 128, 1 << 20, 1 << 20, split_slots=1 << 16)
    assert jfa.jfa_workspace_bytes(p, 0) > jfa._lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(jfa.JfaError) as e:
        jfa.jfa_forward_noalloc(p, 256, 256, 256, None, None, None, 256, 256, None, 256, 256)
    assert e.value.status == jfa._lib.JFA_ERR_WORKSPACE
