"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Sizes are small enough for the oracle to finish in seconds yet span several query and key
tiles, ragged tails, empty samples and asymmetric lengths.
"""
import numpy as np
import pytest
import torch

import oracle
from jfa_synth import custom_case
from tests.gpu_helpers import (compare, compare_lse, device_case, gpu_backward, gpu_forward, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


# ------------------------------------------------------------ offsets

def test_lengths_to_offsets_bitexact():
    import jagged_attention_amd as jfa
    rng = np.random.default_rng(1)
    for B in (1, 5, 1023, 1024, 1025, 3000):
        lens = rng.integers(0, 5000, size=B).astype(np.int32)
        lens[rng.integers(0, B)] = 0
        off, st = jfa.lengths_to_offsets(torch.as_tensor(lens).cuda())
        assert int(st.item()) == 0
        want = oracle.offsets(lens)
        assert np.array_equal(off.cpu().numpy().astype(np.int64), want), B
    off, st = jfa.lengths_to_offsets(torch.tensor([3, -1, 2], dtype=torch.int32).cuda())
    assert int(st.item()) == jfa._lib.JFA_ERR_DEVICE_DATA


@pytest.mark.parametrize("asym", [False, True])
def test_bias_offsets_bitexact(asym):
    """Row offsets and the int64 dense-bias block offsets (running sum of q_len * kv_len) against
    the oracle, including totals far beyond 2^31 elements."""
    import jagged_attention_amd as jfa
    rng = np.random.default_rng(2 + asym)
    for B in (1, 7, 1025, 3000):
        ql = rng.integers(0, 5000, size=B).astype(np.int32)
        kl = rng.integers(0, 5000, size=B).astype(np.int32) if asym else ql
        ql[rng.integers(0, B)] = 0
        off, boff, st = jfa.bias_offsets(torch.as_tensor(ql).cuda(),
                                         torch.as_tensor(kl).cuda() if asym else None)
        assert int(st.item()) == 0
        assert np.array_equal(off.cpu().numpy().astype(np.int64), oracle.offsets(ql)), B
        want = oracle.bias_offsets(ql, kl)
        assert np.array_equal(boff.cpu().numpy(), want), B
        if B == 3000:
            assert want[-1] > 2 ** 31
    # a negative kv length is malformed: status set, neither array written
    off = torch.full((4,), 7, dtype=torch.int32).cuda()
    boff = torch.full((4,), 7, dtype=torch.int64).cuda()
    st = torch.zeros(1, dtype=torch.int32).cuda()
    jfa.jfa_lengths_to_offsets(torch.tensor([3, 1, 2], dtype=torch.int32).cuda(), 3, off, boff,
                               torch.tensor([3, -1, 2], dtype=torch.int32).cuda(), st)
    assert int(st.item()) == jfa._lib.JFA_ERR_DEVICE_DATA
    assert off.cpu().tolist() == [7] * 4 and boff.cpu().tolist() == [7] * 4


# ------------------------------------------------------------ tile lists

SCHED_BATCHES = [
    ([300, 0, 70, 129], [300, 0, 70, 129], True),
    ([1024], [1024], True),
    ([5, 64, 65, 128, 129, 1, 0, 700], [9, 3, 64, 0, 250, 77, 5, 700], False),
    ([5, 64, 65, 128, 129, 1, 0, 700], [9, 3, 64, 0, 250, 77, 5, 700], True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bi", range(len(SCHED_BATCHES)))
@pytest.mark.parametrize("slots", [0, -1, 7, 64])
def test_schedule_bitexact(dtype, bi, slots):
    import jagged_attention_amd as jfa
    ql, kl, causal = SCHED_BATCHES[bi]
    ql, kl = np.array(ql, np.int32), np.array(kl, np.int32)
    H = 3
    p = jfa.make_problem(len(ql), H, 128 if dtype == "bf16" else 64, int(ql.sum()), int(kl.sum()),
                         dtype=dtype, causal=causal, split_slots=slots)
    tc = jfa.jfa_tile_config(p)
    qo = torch.as_tensor(oracle.offsets(ql).astype(np.int32)).cuda()
    ko = torch.as_tensor(oracle.offsets(kl).astype(np.int32)).cuda()
    got = jfa.build_schedule(p, qo, ko)
    want = oracle.schedule(oracle.offsets(ql), oracle.offsets(kl), H, causal, bm=tc["bm"],
                           bn=tc["bn"], slots=tc["slots"], bq_bm=tc["bq_bm"], bq_bn=tc["bq_bn"],
                           bk_bn=tc["bk_bn"], bk_bm=tc["bk_bm"], fuse=int(tc["fuse"]))
    assert got["status"] == 0
    assert np.array_equal(got["fwd"].numpy(), want["fwd"])
    assert np.array_equal(got["fwd_slot"].numpy(), want["fwd_slot"])
    assert np.array_equal(got["combine"].numpy(), want["combine"])
    assert np.array_equal(got["bwd_q"].numpy(), want["bwd_q"])
    assert np.array_equal(got["bwd_kv"].numpy(), want["bwd_kv"])
    assert got["split_threshold"] == want["split_threshold"]


def test_schedule_large_list_global_sort():
    """More records than the LDS sort holds: the global-memory sort path."""
    import jagged_attention_amd as jfa
    rng = np.random.default_rng(5)
    ql = rng.integers(1, 400, size=6000).astype(np.int32)
    p = jfa.make_problem(len(ql), 2, 128, int(ql.sum()), int(ql.sum()), causal=True,
                         split_slots=-1)
    tc = jfa.jfa_tile_config(p)
    off = oracle.offsets(ql)
    got = jfa.build_schedule(p, torch.as_tensor(off.astype(np.int32)).cuda(),
                             torch.as_tensor(off.astype(np.int32)).cuda())
    want = oracle.schedule(off, off, 2, True, bm=tc["bm"], bn=tc["bn"], slots=tc["slots"],
                           bq_bm=tc["bq_bm"], bq_bn=tc["bq_bn"], bk_bn=tc["bk_bn"],
                           bk_bm=tc["bk_bm"], fuse=int(tc["fuse"]))
    assert len(want["fwd"]) > 8192
    assert np.array_equal(got["fwd"].numpy(), want["fwd"])
    assert np.array_equal(got["bwd_kv"].numpy(), want["bwd_kv"])


def test_schedule_rejects_bad_offsets():
    import jagged_attention_amd as jfa
    p = jfa.make_problem(3, 1, 128, 10, 10)
    bad = torch.tensor([0, 6, 4, 10], dtype=torch.int32).cuda()
    got = jfa.build_schedule(p, bad, bad)
    assert got["status"] == jfa._lib.JFA_ERR_DEVICE_DATA
    assert len(got["fwd"]) == 0


# ------------------------------------------------------- forward/backward

PARITY = [
    # q_lens, kv_lens, H, d
    ([300, 17, 129, 0, 64, 200], None, 2, 128),
    ([33, 190, 1, 64, 65], [70, 20, 130, 0, 64], 2, 64),
    ([256, 40, 256], [8, 64, 37], 2, 64),
]


@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal,bias_kind", [(False, "none"), (True, "relpos"),
                                              (False, "dense"), (True, "none"),
                                              (False, "relpos")])
@pytest.mark.parametrize("pi", range(len(PARITY)))
def test_parity_bf16(mode, causal, bias_kind, pi):
    """bf16 forward and backward against the oracle.  Non-causal with a relative-position table
    covers pairs past a sample's end whose bias is not zero: the GDPA kernels leave them
    unmasked, relying on their K and V rows reading as zero."""
    ql, kl, H, d = PARITY[pi]
    kl = ql if kl is None else kl
    case = custom_case(ql, kl, H, d, dtype="bf16", mode=mode, causal=causal, bias_kind=bias_kind,
                       seed=10 + pi)
    say(f"[parity bf16] mode={mode} causal={causal} bias={bias_kind} case={pi}")
    o, lse, dc = gpu_forward(case)
    o_ref, lse_ref = oracle.case_forward(case)
    compare("O", o, o_ref, "bf16")
    if mode == "softmax":
        compare_lse(lse, lse_ref, mode)
    dq, dk, dv = gpu_backward(case, o, lse, dc)
    dq_ref, dk_ref, dv_ref = oracle.case_backward(case)
    compare("dQ", dq, dq_ref, "bf16")
    compare("dK", dk, dk_ref, "bf16")
    compare("dV", dv, dv_ref, "bf16")


@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal,bias_kind", [(False, "none"), (True, "relpos"), (False, "dense")])
def test_parity_f32(mode, causal, bias_kind):
    ql = [100, 0, 128, 7]
    case = custom_case(ql, [90, 12, 128, 7] if not causal else ql, 2, 64, dtype="f32", mode=mode,
                       causal=causal, bias_kind=bias_kind, seed=3)
    say(f"[parity f32] mode={mode} causal={causal} bias={bias_kind}")
    o, lse, dc = gpu_forward(case)
    o_ref, lse_ref = oracle.case_forward(case)
    compare("O", o, o_ref, "f32")
    compare_lse(lse, lse_ref, mode, tol=1e-5)
    dq, dk, dv = gpu_backward(case, o, lse, dc)
    dq_ref, dk_ref, dv_ref = oracle.case_backward(case)
    compare("dQ", dq, dq_ref, "f32")
    compare("dK", dk, dk_ref, "f32")
    compare("dV", dv, dv_ref, "f32")


@pytest.mark.parametrize("mode", ["softmax", "silu"])
def test_split_kv_forward(mode):
    """Long causal samples with a small slot count force split tiles and the combine pass."""
    case = custom_case([1500, 40, 900], [1500, 40, 900], 2, 128, dtype="bf16", mode=mode,
                       causal=True, bias_kind="relpos", seed=21, with_dout=False)
    say(f"[split] mode={mode}")
    o, lse, _ = gpu_forward(case, split_slots=4)
    o_ref, lse_ref = oracle.case_forward(case)
    compare("O", o, o_ref, "bf16")
    compare_lse(lse, lse_ref, mode)
    o2, lse2, _ = gpu_forward(case, split_slots=-1)
    compare("O(no split)", o2, o_ref, "bf16")


def test_zero_length_samples_bf16():
    ql = [0, 5, 0, 70]
    kl = [3, 0, 0, 64]
    for mode in ("softmax", "gelu"):
        case = custom_case(ql, kl, 2, 128, dtype="bf16", mode=mode, seed=4)
        o, lse, dc = gpu_forward(case)
        assert torch.all(o[0:5] == 0)                    # sample 1 has no keys
        if mode == "softmax":
            assert torch.all(torch.isneginf(lse[:, 0:5]))
        dq, dk, dv = gpu_backward(case, o, lse, dc)
        assert torch.all(dq[0:5] == 0)
        assert torch.all(dk[0:3] == 0) and torch.all(dv[0:3] == 0)   # sample 0 has no queries
        o_ref, _ = oracle.case_forward(case)
        compare("O", o, o_ref, "bf16")


def test_backward_deterministic():
    case = custom_case([400, 77, 129], [400, 77, 129], 2, 128, dtype="bf16", causal=True,
                       bias_kind="relpos", seed=9)
    o, lse, dc = gpu_forward(case)
    a = gpu_backward(case, o, lse, dc)
    b = gpu_backward(case, o, lse, dc)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    o2, lse2, _ = gpu_forward(case, dc)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


# ------------------------------------------------------------------ MXFP8

def test_mxfp8_quantizer_bitexact():
    import jagged_attention_amd as jfa
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal((777, 4, 128), dtype=np.float32)).to(torch.bfloat16)
    x[3, 1, :32] = 0
    x[5, 2, 32:64] *= 1e-20
    x[6, 0, 64:96] *= 300.0
    codes, scales = jfa.quantize_mxfp8(x.cuda())
    want_c, want_s = oracle.mxfp8_quantize(x.double().numpy())
    assert np.array_equal(scales.cpu().numpy(), want_s)
    assert np.array_equal(codes.cpu().numpy(), want_c)


def test_mxfp8_quantizer_batch_matches_single():
    import jagged_attention_amd as jfa
    rng = np.random.default_rng(31)
    shapes = [(1000, 4, 128), (3, 4, 128), (0, 4, 128), (40000, 4, 128)]   # the last: two
    # grid-stride iterations (the grid is capped at 8 workgroups per CU)
    xs = [torch.from_numpy((rng.standard_normal(s) * np.exp(rng.normal(0, 3, s[:2] + (1,))))
                           .astype(np.float32)).to(torch.bfloat16).cuda() for s in shapes]
    d = 128
    codes = [torch.full(x.shape, 0x5A, dtype=torch.uint8, device="cuda") for x in xs]
    scales = [torch.full(tuple(x.shape[:-1]) + (d // 32,), 0x5A, dtype=torch.uint8,
                         device="cuda") for x in xs]
    jfa.jfa_quantize_mxfp8_batch(xs, [x.numel() // d for x in xs], d, codes, scales)
    torch.cuda.synchronize()
    for x, c, s in zip(xs, codes, scales):
        wc, ws = jfa.quantize_mxfp8(x)
        assert torch.equal(c, wc) and torch.equal(s, ws)
    # and against the oracle on one of them
    want_c, want_s = oracle.mxfp8_quantize(xs[0].cpu().double().numpy())
    assert np.array_equal(codes[0].cpu().numpy(), want_c)
    assert np.array_equal(scales[0].cpu().numpy(), want_s)


def test_mxfp8_quantizer_golden():
    """The hand-derived cases (ties to even, smallest subnormal, saturation, zero block) on the
    GPU quantiser: one 32-element block per case holding amax and x."""
    import jagged_attention_amd as jfa
    from tests.test_oracle_pins import _golden_rows
    rows = list(_golden_rows("mxfp8_cases.txt"))
    blk = np.zeros((len(rows), 32), dtype=np.float32)
    for r, (amax, x, _, _) in enumerate(rows):
        blk[r, 0], blk[r, 1] = float(amax), float(x)
        blk[r, 2] = -float(x)                      # the same magnitude, the other sign
    xb = torch.from_numpy(blk).to(torch.bfloat16)
    # every x is bf16-exact; an amax may round, but not across a power of two (same scale)
    assert torch.equal(xb[:, 1:].float(), torch.from_numpy(blk[:, 1:]))
    a0 = xb[:, 0].float().numpy()
    nz = blk[:, 0] > 0
    assert np.array_equal(np.floor(np.log2(a0[nz])), np.floor(np.log2(blk[nz, 0])))
    codes, scales = jfa.quantize_mxfp8(xb.cuda())
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    for r, (amax, x, scale, code) in enumerate(rows):
        c = int(code, 16)
        assert scales[r, 0] == int(scale), (amax, x)
        assert codes[r, 1] == c, (amax, x, hex(codes[r, 1]))
        if float(amax) != 0.0:
            assert codes[r, 2] == (c ^ 0x80), (amax, x, hex(codes[r, 2]))


def test_mxfp8_forward_parity():
    import jagged_attention_amd as jfa
    ql = [300, 17, 129, 0, 64, 520]
    case = custom_case(ql, ql, 2, 128, dtype="mxfp8", causal=True, seed=31, with_dout=False)
    dc = device_case(case)
    qc, qs = jfa.quantize_mxfp8(dc["q"])
    kc, ks = jfa.quantize_mxfp8(dc["k"])
    vc, vs = jfa.quantize_mxfp8(dc["v"])
    o, lse = jfa.forward(qc, kc, vc, dc["qo"], dc["ko"], causal=True, q_scale=qs, k_scale=ks,
                         v_scale=vs)
    torch.cuda.synchronize()
    deq = [oracle.mxfp8_dequantize(c.cpu().numpy(), s.cpu().numpy()) for c, s in
           ((qc, qs), (kc, ks), (vc, vs))]
    o_ref, lse_ref = oracle.forward(deq[0], deq[1], deq[2], case.q_lens, case.kv_lens,
                                    causal=True)
    from tests.helpers import rel_l2
    rl = rel_l2(o.float().cpu().numpy(), o_ref)
    say(f"[mxfp8] rel-L2 {rl:.3g}")
    assert rl <= 5e-2
    compare_lse(lse, lse_ref, "softmax", tol=1e-2)


def test_mxfp8_forward_block_scales_differ():
    """Every 32-element block along d gets its own power-of-two magnitude, so each row's
    E8M0 scales differ block to block: a scale applied to the wrong block shows up."""
    import jagged_attention_amd as jfa
    ql = [200, 1, 77, 130]
    case = custom_case(ql, ql, 2, 128, dtype="mxfp8", causal=True, seed=41, with_dout=False)
    rng = np.random.default_rng(42)
    dc = device_case(case)
    scaled = []
    for name in ("q", "k", "v"):
        x = dc[name]
        e = rng.integers(-4, 5, size=(x.shape[0], x.shape[1], x.shape[2] // 32))
        f = torch.from_numpy(np.exp2(e).astype(np.float32)).repeat_interleave(32, dim=2)
        scaled.append((x.float().cpu() * f).to(torch.bfloat16).cuda())
    qs8 = [jfa.quantize_mxfp8(x) for x in scaled]
    o, lse = jfa.forward(qs8[0][0], qs8[1][0], qs8[2][0], dc["qo"], dc["ko"], causal=True,
                         q_scale=qs8[0][1], k_scale=qs8[1][1], v_scale=qs8[2][1])
    torch.cuda.synchronize()
    deq = [oracle.mxfp8_dequantize(c.cpu().numpy(), s.cpu().numpy()) for c, s in qs8]
    for (c, s), x in zip(qs8, scaled):
        # the per-block scales really differ within rows
        sv = s.cpu().numpy().astype(np.int64)
        assert (sv.max(axis=2) - sv.min(axis=2)).max() >= 4
    o_ref, lse_ref = oracle.forward(deq[0], deq[1], deq[2], case.q_lens, case.kv_lens,
                                    causal=True)
    from tests.helpers import rel_l2
    rl = rel_l2(o.float().cpu().numpy(), o_ref)
    say(f"[mxfp8 block scales] rel-L2 {rl:.3g}")
    assert rl <= 5e-2
    compare_lse(lse, lse_ref, "softmax", tol=2e-2)
