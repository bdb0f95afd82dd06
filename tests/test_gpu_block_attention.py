"""GPU parity for BlockAttention: the library's refined offsets (bit-exact against the oracle's
block list) fed to the jagged kernels, against the oracle's block-diagonal attention on the
original samples."""
import numpy as np
import pytest
import torch

import oracle
from jfa_synth import custom_case
from tests.gpu_helpers import compare, compare_lse, device_case, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


def _refined(dc, case, w):
    import jagged_attention_amd as jfa
    boff, nb, st = jfa.block_offsets(dc["qo"], w, case.total_q)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    qo = np.concatenate([[0], np.cumsum(case.q_lens.astype(np.int64))])
    want = oracle.block_offsets(qo, w)
    assert np.array_equal(boff.cpu().numpy().astype(np.int64), want)
    return boff, nb


@pytest.mark.parametrize("w", [64, 100, 256])
def test_block_offsets_bitexact(w):
    lens = [300, 17, 129, 0, 64, 200, 1, 4096]
    case = custom_case(lens, lens, 1, 64, dtype="bf16", seed=5, with_dout=False)
    say(f"[block offsets] w={w}")
    _refined(device_case(case), case, w)


def test_block_offsets_rejects_small_batch():
    import jagged_attention_amd as jfa
    off = torch.tensor([0, 10, 10, 25], dtype=torch.int32).cuda()
    out = torch.full((4,), -7, dtype=torch.int32).cuda()
    st = torch.zeros(1, dtype=torch.int32).cuda()
    jfa.jfa_block_offsets(off, 3, 4, out, 3, st)      # needs 3 + 4 = 7 blocks
    torch.cuda.synchronize()
    assert int(st.item()) == jfa._lib.JFA_ERR_DEVICE_DATA
    assert torch.all(out == -7)                        # nothing written
    bad = torch.tensor([0, 10, 5, 25], dtype=torch.int32).cuda()
    big = torch.full((21,), -7, dtype=torch.int32).cuda()
    jfa.jfa_block_offsets(bad, 3, 4, big, 20, st)
    torch.cuda.synchronize()
    assert int(st.item()) == jfa._lib.JFA_ERR_DEVICE_DATA


@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal,bias_kind", [(True, "relpos"), (False, "none")])
@pytest.mark.parametrize("w,d", [(64, 128), (100, 128), (256, 64)])
def test_block_attention_parity(mode, causal, bias_kind, w, d):
    import jagged_attention_amd as jfa
    lens = [300, 17, 129, 0, 64, 700]
    case = custom_case(lens, lens, 2, d, dtype="bf16", mode=mode, causal=causal,
                       bias_kind=bias_kind, seed=40 + w)
    say(f"[block attention] mode={mode} causal={causal} bias={bias_kind} w={w} d={d}")
    dc = device_case(case)
    boff, nb = _refined(dc, case, w)
    kw = dict(mode=mode, causal=causal, bias=dc["bias"], bias_kind=bias_kind,
              num_buckets=case.num_buckets)
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], boff, boff, **kw)
    dq, dk, dv = jfa.backward(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], boff, boff, **kw)
    torch.cuda.synchronize()
    okw = dict(mode=mode, causal=causal, bias=case.bias, bias_kind=bias_kind,
               num_buckets=case.num_buckets, block=w)
    o_ref, lse_ref = oracle.forward(case.q, case.k, case.v, case.q_lens, case.kv_lens, **okw)
    dq_ref, dk_ref, dv_ref = oracle.backward(case.q, case.k, case.v, case.dout, case.q_lens,
                                             case.kv_lens, **okw)
    compare("O", o, o_ref, "bf16")
    compare_lse(lse, lse_ref, mode)
    compare("dQ", dq, dq_ref, "bf16")
    compare("dK", dk, dk_ref, "bf16")
    compare("dV", dv, dv_ref, "bf16")
