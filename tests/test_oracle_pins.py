"""Pins the fp64 oracle to things other than itself.

Each check here would fail on a plausible mistake in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong mask alignment):
  - torch's own scaled_dot_product_attention / autograd / silu / gelu (fp64);
  - a dense, padded, batched computation (jagged must equal masked-padded);
  - central finite differences of the forward;
  - closed forms and hand-computed fixtures under tests/golden/;
  - brute-force enumeration of tile lists;
  - torch's float8_e4m3fn for the E4M3 code table.
"""
import math
import os

import numpy as np
import pytest
import torch

from jfa_synth import custom_case
from tests.conftest import GOLDEN
from tests.helpers import max_abs, rel_l2, torch_reference

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


# ------------------------------------------------------------------ offsets

def test_offsets_match_cumsum(oracle_mod):
    rng = np.random.default_rng(0)
    for _ in range(20):
        lens = rng.integers(0, 1000, size=rng.integers(1, 50)).astype(np.int32)
        off = oracle_mod.offsets(lens)
        assert off.dtype == np.int64
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(lens.astype(np.int64))]))


def test_offsets_reject_negative(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.offsets(np.array([3, -1, 2], np.int32))


def test_bias_offsets_are_running_products(oracle_mod):
    q = np.array([3, 0, 5, 7], np.int32)
    kv = np.array([2, 4, 0, 9], np.int32)
    assert list(oracle_mod.bias_offsets(q, kv)) == [0, 6, 6, 6, 69]


# ------------------------------------------------------- relative position

def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_relpos_bucket_golden(oracle_mod):
    rows = _golden_rows("relpos_buckets.txt")
    assert len(rows) >= 20
    for dist, width, want in rows:
        assert oracle_mod.relpos_bucket(int(dist), int(width)) == int(want), (dist, width)


def test_relpos_bucket_invariants(oracle_mod):
    prev = 0
    for d in range(0, 70000):
        bkt = oracle_mod.relpos_bucket(d, 64)
        assert prev <= bkt <= 63
        prev = bkt
    # four buckets per doubling between 16 and 2^15
    for k in range(4, 15):
        seen = {oracle_mod.relpos_bucket(d, 64) for d in range(2 ** k, 2 ** (k + 1))}
        assert len(seen) == 4


# -------------------------------------------------------- worked example

def test_worked_example(oracle_mod):
    s2 = math.sqrt(2.0)
    q = np.array([[[0.0, 0.0]], [[s2 * math.log(3.0), 0.0]]])
    k = np.array([[[1.0, 0.0]], [[0.0, 0.0]]])
    v = np.array([[[4.0, 8.0]], [[0.0, 4.0]]])
    lens = np.array([2], np.int32)
    for mode, causal, row, o0, o1, lse in _golden_rows("attention_worked_example.txt"):
        ev = lambda s: eval(s, {"log": math.log, "nan": float("nan")})  # noqa: E731
        o, l = oracle_mod.forward(q, k, v, lens, lens, mode=mode, causal=bool(int(causal)))
        r = int(row)
        assert abs(o[r, 0, 0] - ev(o0)) < 1e-12 and abs(o[r, 0, 1] - ev(o1)) < 1e-12
        if mode == "softmax":
            assert abs(l[0, r] - ev(lse)) < 1e-12


# ------------------------------------------- attention vs torch (fp64)

CASES = [
    # q_lens, kv_lens, H, d
    ([5, 0, 9, 1, 12], [5, 0, 9, 1, 12], 2, 16),
    ([4, 7, 3], [9, 2, 3], 2, 8),           # asymmetric, q longer and shorter than kv
    ([6, 3], [0, 5], 1, 8),                  # an empty key set
]


@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bias_kind", ["none", "relpos", "dense"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_forward_backward_vs_torch(oracle_mod, mode, causal, bias_kind, ci):
    ql, kl, H, d = CASES[ci]
    case = custom_case(ql, kl, H, d, dtype="f32", mode=mode, causal=causal,
                       bias_kind=bias_kind, num_buckets=64, seed=100 + ci, bias_std=0.5)
    o, lse = oracle_mod.case_forward(case)
    dq, dk, dv = oracle_mod.case_backward(case)
    ref = torch_reference(case.q, case.k, case.v, case.q_lens, case.kv_lens, mode, causal,
                          case.bias, bias_kind, oracle_mod.relpos_bucket, dout=case.dout)
    assert max_abs(o, ref["o"]) < 1e-12
    if mode == "softmax":
        finite = np.isfinite(ref["lse"])
        assert np.array_equal(np.isfinite(lse), finite)
        assert np.all(lse[~finite] == -np.inf)
        assert max_abs(lse[finite], ref["lse"][finite]) < 1e-12
    else:
        assert lse is None
    for got, want in ((dq, ref["dq"]), (dk, ref["dk"]), (dv, ref["dv"])):
        assert max_abs(got, want) < 1e-11


def test_jagged_equals_masked_padded(oracle_mod):
    """A padded, batched torch computation with a key-padding mask agrees on valid rows."""
    ql = np.array([7, 3, 11, 1], np.int32)
    kl = np.array([9, 3, 4, 6], np.int32)
    H, d = 3, 8
    for mode in ("softmax", "silu"):
        case = custom_case(ql, kl, H, d, dtype="f32", mode=mode, seed=7)
        o, _ = oracle_mod.case_forward(case)
        B, Lq, Lk = len(ql), int(ql.max()), int(kl.max())
        qp = torch.zeros(B, H, Lq, d, dtype=torch.float64)
        kp = torch.zeros(B, H, Lk, d, dtype=torch.float64)
        vp = torch.zeros(B, H, Lk, d, dtype=torch.float64)
        qo = np.concatenate([[0], np.cumsum(ql)])
        ko = np.concatenate([[0], np.cumsum(kl)])
        for b in range(B):
            qp[b, :, :ql[b]] = case.q[qo[b]:qo[b + 1]].double().permute(1, 0, 2)
            kp[b, :, :kl[b]] = case.k[ko[b]:ko[b + 1]].double().permute(1, 0, 2)
            vp[b, :, :kl[b]] = case.v[ko[b]:ko[b + 1]].double().permute(1, 0, 2)
        s = (qp @ kp.transpose(-1, -2)) / math.sqrt(d)
        keymask = torch.arange(Lk)[None, :] < torch.as_tensor(kl)[:, None]   # [B, Lk]
        if mode == "softmax":
            s = s.masked_fill(~keymask[:, None, None, :], -math.inf)
            op = torch.softmax(s, dim=-1) @ vp
        else:
            a = torch.nn.functional.silu(s) * keymask[:, None, None, :]
            # the true kv_len divides, never the padded length
            op = (a @ vp) / torch.as_tensor(kl, dtype=torch.float64)[:, None, None, None]
        for b in range(B):
            got = o[qo[b]:qo[b + 1]]
            want = op[b, :, :ql[b]].permute(1, 0, 2).numpy()
            assert max_abs(got, want) < 1e-12


# ---------------------------------------------------- finite differences

@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal,bias_kind", [(False, "none"), (True, "relpos"), (False, "dense")])
def test_backward_central_differences(oracle_mod, mode, causal, bias_kind):
    ql, kl = [3, 6, 2], [4, 6, 5]
    case = custom_case(ql, kl, 2, 4, dtype="f32", mode=mode, causal=causal, bias_kind=bias_kind,
                       seed=11, bias_std=0.5)
    q, k, v = (case.q.double().numpy().copy() for _ in range(1)), None, None
    q = case.q.double().numpy().copy()
    k = case.k.double().numpy().copy()
    v = case.v.double().numpy().copy()
    dout = case.dout.double().numpy()
    kw = dict(mode=mode, causal=causal, bias=case.bias, bias_kind=bias_kind)

    def loss(qq, kk, vv):
        o, _ = oracle_mod.forward(qq, kk, vv, case.q_lens, case.kv_lens, **kw)
        return float(np.sum(o * dout))

    dq, dk, dv = oracle_mod.backward(q, k, v, dout, case.q_lens, case.kv_lens, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = loss(q, k, v)
            x[idx] = old - h
            lm = loss(q, k, v)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - g)) / max(1.0, np.max(np.abs(g)))
        assert err < 1e-6, (name, err)


# ----------------------------------------------------------- closed forms

def test_closed_forms_softmax(oracle_mod):
    ql = np.array([6, 4, 1], np.int32)
    for causal in (False, True):
        case = custom_case(ql, ql, 2, 8, dtype="f32", causal=causal, seed=3)
        # V = 1 -> O = 1 (the weights of every row sum to one)
        o, _ = oracle_mod.forward(case.q, case.k, torch.ones_like(case.v), ql, ql, causal=causal)
        assert max_abs(o, np.ones_like(o)) < 1e-13
        # K = 0, no bias -> O_i = mean of the visible V_j (prefix mean when causal)
        o, lse = oracle_mod.forward(case.q, torch.zeros_like(case.k), case.v, ql, ql,
                                    causal=causal)
        v = case.v.double().numpy()
        off = 0
        for n in ql:
            for i in range(n):
                upto = i + 1 if causal else n
                want = v[off:off + upto].mean(axis=0)
                assert max_abs(o[off + i], want) < 1e-13
                assert abs(lse[0, off + i] - math.log(upto)) < 1e-13
            off += n
    # kv_len = 1 -> O_i = V_0, and dQ = dK = 0 exactly
    case = custom_case([5, 3], [1, 1], 2, 8, dtype="f32", seed=4)
    o, _ = oracle_mod.case_forward(case)
    dq, dk, dv = oracle_mod.case_backward(case)
    v = case.v.double().numpy()
    assert max_abs(o[:5], np.broadcast_to(v[0], (5, 2, 8))) < 1e-14
    assert max_abs(o[5:], np.broadcast_to(v[1], (3, 2, 8))) < 1e-14
    assert np.all(dq == 0) and np.all(dk == 0)
    # a per-row constant added to a dense bias leaves softmax output unchanged
    case = custom_case([4, 5], [6, 3], 2, 8, dtype="f32", bias_kind="dense", seed=5)
    o1, _ = oracle_mod.case_forward(case)
    shifted = case.bias.double().clone()
    off = 0
    for n, m in zip(case.q_lens, case.kv_lens):
        blk = shifted[off:off + 2 * n * m].view(2, n, m)
        blk += torch.arange(n, dtype=torch.float64)[None, :, None] * 3.0
        off += 2 * n * m
    o2, _ = oracle_mod.forward(case.q, case.k, case.v, case.q_lens, case.kv_lens,
                               bias=shifted, bias_kind="dense")
    assert max_abs(o1, o2) < 1e-13


@pytest.mark.parametrize("mode", ["silu", "gelu"])
def test_closed_forms_gdpa(oracle_mod, mode):
    ql, kl = np.array([4, 3], np.int32), np.array([5, 2], np.int32)
    case = custom_case(ql, kl, 2, 8, dtype="f32", mode=mode, seed=6)
    # Q = 0, no bias -> every score is 0 and act(0) = 0 -> O = 0
    o, _ = oracle_mod.forward(torch.zeros_like(case.q), case.k, case.v, ql, kl, mode=mode)
    assert np.all(o == 0)
    # K = 0 -> scores 0, act'(0) = 1/2: dK_j = (s / (2 m)) sum_i (dO_i . V_j) Q_i
    dq, dk, dv = oracle_mod.backward(case.q, torch.zeros_like(case.k), case.v, case.dout, ql, kl,
                                     mode=mode)
    q, v, do = (t.double().numpy() for t in (case.q, case.v, case.dout))
    s = 1 / math.sqrt(8)
    qoff = koff = 0
    for n, m in zip(ql, kl):
        for h in range(2):
            for j in range(m):
                want = sum((do[qoff + i, h] @ v[koff + j, h]) * q[qoff + i, h] for i in range(n))
                want = want * s / (2 * m)
                assert max_abs(dk[koff + j, h], want) < 1e-13
        qoff += n
        koff += m


def test_zero_length_samples(oracle_mod):
    ql = np.array([3, 0, 4, 2], np.int32)
    kl = np.array([0, 5, 3, 2], np.int32)
    for mode in ("softmax", "silu", "gelu"):
        case = custom_case(ql, kl, 2, 8, dtype="f32", mode=mode, seed=8)
        o, lse = oracle_mod.case_forward(case)
        dq, dk, dv = oracle_mod.case_backward(case)
        assert np.all(o[:3] == 0) and np.all(dq[:3] == 0)       # sample 0 has no keys
        if mode == "softmax":
            assert np.all(lse[:, :3] == -np.inf)
        assert np.all(dk[:5] == 0) and np.all(dv[:5] == 0)      # sample 1 has no queries
        assert np.any(o[3:] != 0)


# -------------------------------------------------------------- tile lists

def _parse_schedule_golden():
    cases, cur = [], None
    for row in _golden_rows("schedule_small.txt"):
        key = row[0]
        if key == "case":
            cur = dict(name=row[1], rec=[], comb=[])
        elif key == "end":
            cases.append(cur)
        elif key in ("rec", "comb"):
            cur[key].append([int(x) for x in row[1:]])
        elif key == "q_lens":
            cur[key] = [int(x) for x in row[1:]]
        else:
            cur[key] = int(row[1])
    return cases


def test_schedule_golden(oracle_mod):
    for c in _parse_schedule_golden():
        off = oracle_mod.offsets(np.array(c["q_lens"], np.int32))
        s = oracle_mod.schedule(off, off, c["heads"], bool(c["causal"]), bm=c["bm"], bn=c["bn"],
                                slots=c["slots"], bq_bm=64, bq_bn=64, bk_bn=64, bk_bm=64)
        got = np.concatenate([s["fwd"], s["fwd_slot"][:, None]], axis=1).tolist()
        assert got == c["rec"], c["name"]
        assert s["combine"].tolist() == c["comb"], c["name"]
        assert s["split_threshold"] == c["threshold"]


def _visible_pairs(n, m, causal, r0, r1, c0, c1):
    cnt = 0
    for i in range(r0, min(r1, n)):
        for j in range(c0, min(c1, m)):
            if not causal or j <= i + (m - n):
                cnt += 1
    return cnt


@pytest.mark.parametrize("seed", range(6))
def test_schedule_invariants_bruteforce(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 12))
    ql = rng.integers(0, 300, size=B).astype(np.int32)
    kl = ql.copy() if seed % 2 == 0 else rng.integers(0, 300, size=B).astype(np.int32)
    causal = seed % 3 != 2
    H, bm, bn = int(rng.integers(1, 5)), 64 * int(rng.integers(1, 3)), 32 * int(rng.integers(1, 3))
    slots = int(rng.integers(1, 40)) if seed != 5 else 0
    qo, ko = oracle_mod.offsets(ql), oracle_mod.offsets(kl)
    s = oracle_mod.schedule(qo, ko, H, causal, bm=bm, bn=bn, slots=slots, bq_bm=64, bq_bn=32,
                            bk_bn=64, bk_bm=32)
    fwd, slot = s["fwd"], s["fwd_slot"]
    cost = np.maximum(1, fwd[:, 3] - fwd[:, 2])
    # longest first, ties by (b, t, kb): the list is sorted by a total order
    keys = [(-c, b, t, kb) for c, (b, t, kb, _) in zip(cost, fwd)]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)
    # every query tile appears; its chunks tile [0, steps) exactly; steps cover every visible pair
    C = s["split_threshold"]
    for b in range(B):
        n, m = int(ql[b]), int(kl[b])
        for t in range(-(-n // bm)):
            parts = sorted([tuple(r[2:]) for r in fwd if r[0] == b and r[1] == t])
            assert parts[0][0] == 0
            for a, c in zip(parts, parts[1:]):
                assert a[1] == c[0]
            steps = parts[-1][1]
            # steps is the smallest count covering every visible pair of the tile
            assert _visible_pairs(n, m, causal, t * bm, (t + 1) * bm, 0, steps * bn) == \
                _visible_pairs(n, m, causal, t * bm, (t + 1) * bm, 0, m)
            if steps > 0:
                assert _visible_pairs(n, m, causal, t * bm, (t + 1) * bm, (steps - 1) * bn,
                                      steps * bn) > 0
            if slots > 0 and steps > C:
                assert len(parts) == -(-steps // C)
            else:
                assert len(parts) == 1
        assert not any(r[0] == b and r[1] >= -(-n // bm) for r in fwd)
    # split chunks own distinct, dense partial slots
    used = sorted(slot[slot >= 0].tolist())
    assert used == list(range(len(used)))
    # backward classes: one query tile -> q-stationary single pass (owns dK/dV);
    # else one key tile -> kv-stationary single pass (owns dQ); else both passes.
    for b in range(B):
        n, m = int(ql[b]), int(kl[b])
        one_q = -(-n // 64) == 1
        one_k = not one_q and -(-m // 64) == 1
        rq = [r for r in s["bwd_q"] if r[0] == b]
        rk = [r for r in s["bwd_kv"] if r[0] == b]
        assert len(rq) == (0 if one_k else -(-n // 64))
        assert len(rk) == (0 if one_q else -(-m // 64))
        if one_q:
            assert rq[0][3] == -(-m // 32)            # visits every key tile
        for _, u, first, end in rk:
            assert end == -(-n // 32)
            if one_k or not causal:
                assert first == 0                     # visits every query tile
            elif first < end:
                # the first query tile is the first one with a visible pair
                assert _visible_pairs(n, m, causal, 0, first * 32, u * 64, (u + 1) * 64) == 0
                assert _visible_pairs(n, m, causal, first * 32, (first + 1) * 32, u * 64,
                                      (u + 1) * 64) > 0
            else:
                assert _visible_pairs(n, m, causal, 0, n, u * 64, (u + 1) * 64) == 0


def test_schedule_rejects_bad_offsets(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.schedule(np.array([0, 5, 3], np.int64), np.array([0, 5, 8], np.int64), 1,
                            False, bm=64, bn=64, slots=0, bq_bm=64, bq_bn=64, bk_bn=64, bk_bm=64)


# ------------------------------------------------------------------ MXFP8

def test_e4m3_table_matches_torch_float8(oracle_mod):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle_mod.e4m3_decode(c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c], c


def test_mxfp8_golden(oracle_mod):
    for amax, x, scale, code in _golden_rows("mxfp8_cases.txt"):
        blk = np.zeros(32)
        blk[0], blk[1] = float(amax), float(x)
        codes, scales = oracle_mod.mxfp8_quantize(blk[None, :])
        assert scales[0, 0] == int(scale), (amax, x)
        assert codes[0, 1] == int(code, 16), (amax, x, hex(codes[0, 1]))


def test_mxfp8_against_torch_cast_and_bounds(oracle_mod):
    rng = np.random.default_rng(9)
    x = torch.from_numpy(rng.standard_normal((512, 128), dtype=np.float32)).to(torch.bfloat16)
    x[3, :32] = 0                                       # an all-zero block
    x[4, 32:64] *= 1e-30                                # tiny magnitudes
    xd = x.double().numpy()
    codes, scales = oracle_mod.mxfp8_quantize(xd)
    deq = oracle_mod.mxfp8_dequantize(codes, scales)
    for r in range(xd.shape[0]):
        for blk in range(4):
            xb = xd[r, 32 * blk:32 * blk + 32]
            amax = np.max(np.abs(xb))
            if amax == 0:
                assert scales[r, blk] == 127 and np.all(codes[r, 32 * blk:32 * blk + 32] == 0)
                continue
            e = int(scales[r, blk]) - 127
            assert 256 <= amax * 2.0 ** -e < 512           # the scale puts amax in the top binade
            y = xb * 2.0 ** -e
            inr = np.abs(y) <= 448
            ref = torch.from_numpy(y[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[r, 32 * blk:32 * blk + 32][inr], ref)
            assert np.all(codes[r, 32 * blk:32 * blk + 32][~inr] & 127 == 0x7E)
            big = (np.abs(y) >= 2.0 ** -6) & inr              # normal, unsaturated E4M3 range
            rel = np.abs(deq[r, 32 * blk:32 * blk + 32][big] - xb[big]) / np.abs(xb[big])
            assert np.all(rel <= 2.0 ** -4)                   # half an ulp of a 3-bit mantissa
            sat = ~inr                                        # y in (448, 512) clips to 448
            rel = np.abs(deq[r, 32 * blk:32 * blk + 32][sat] - xb[sat]) / np.abs(xb[sat])
            assert np.all(rel < 1.0 / 8)


# ------------------------------------------------------------ BlockAttention

def _split_lengths(lens, w):
    """Block lengths of each sample, written out by hand: full blocks of w, then the rest."""
    out = []
    for n in lens:
        n = int(n)
        out += [w] * (n // w) + ([n % w] if n % w else [])
    return out


def test_block_offsets_bruteforce(oracle_mod):
    rng = np.random.default_rng(7)
    for _ in range(50):
        B = int(rng.integers(1, 9))
        lens = rng.integers(0, 40, size=B)
        w = int(rng.integers(1, 17))
        off = np.concatenate([[0], np.cumsum(lens)])
        got = oracle_mod.block_offsets(off, w)
        blocks = _split_lengths(lens, w)
        want = np.concatenate([[0], np.cumsum(blocks)])
        nb = len(blocks)
        assert nb <= B + int(off[-1]) // w              # the documented bound holds
        assert got.shape[0] == B + int(off[-1]) // w + 1
        assert np.array_equal(got[:nb + 1], want)
        assert np.all(got[nb:] == off[-1])              # trailing empty blocks
    with pytest.raises(ValueError):
        oracle_mod.block_offsets([0, 10], 3, out_batch=3)   # needs 4 blocks


@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal,bias_kind", [(False, "none"), (True, "relpos")])
def test_block_attention_is_attention_per_block(oracle_mod, mode, causal, bias_kind):
    """BlockAttention over samples = plain attention (torch SDPA / autograd) over every block
    taken as a sample of its own."""
    lens, w = [11, 0, 4, 9], 4
    case = custom_case(lens, lens, 2, 8, dtype="f32", mode=mode, causal=causal,
                       bias_kind=bias_kind, num_buckets=64, seed=31, bias_std=0.5)
    o, lse = oracle_mod.forward(case.q, case.k, case.v, lens, lens, mode=mode, causal=causal,
                                bias=case.bias, bias_kind=bias_kind, block=w)
    dq, dk, dv = oracle_mod.backward(case.q, case.k, case.v, case.dout, lens, lens, mode=mode,
                                     causal=causal, bias=case.bias, bias_kind=bias_kind, block=w)
    blocks = _split_lengths(lens, w)
    ref = torch_reference(case.q, case.k, case.v, blocks, blocks, mode, causal, case.bias,
                          bias_kind, oracle_mod.relpos_bucket, dout=case.dout)
    assert max_abs(o, ref["o"]) < 1e-12
    if mode == "softmax":
        assert max_abs(lse, ref["lse"]) < 1e-12
    for got, want in ((dq, ref["dq"]), (dk, ref["dk"]), (dv, ref["dv"])):
        assert max_abs(got, want) < 1e-11
    # blocks do change the result (the test would pass vacuously otherwise)
    o_full, _ = oracle_mod.forward(case.q, case.k, case.v, lens, lens, mode=mode, causal=causal,
                                   bias=case.bias, bias_kind=bias_kind)
    assert max_abs(o, o_full) > 1e-3


def test_block_attention_special_cases(oracle_mod):
    lens = [7, 3, 12]
    case = custom_case(lens, lens, 2, 8, dtype="f32", mode="softmax", causal=False, seed=32)
    # a block as long as the longest sample is full attention, bit for bit
    o_w, lse_w = oracle_mod.forward(case.q, case.k, case.v, lens, lens, block=12)
    o_f, lse_f = oracle_mod.forward(case.q, case.k, case.v, lens, lens)
    assert np.array_equal(o_w, o_f) and np.array_equal(lse_w, lse_f)
    # one-row blocks: every query sees only its own key, so O = V, and the softmax weight is
    # constant 1, so dQ = dK = 0 and dV = dO
    o1, _ = oracle_mod.forward(case.q, case.k, case.v, lens, lens, block=1)
    assert max_abs(o1, np.asarray(case.v, np.float64)) < 1e-15
    dq, dk, dv = oracle_mod.backward(case.q, case.k, case.v, case.dout, lens, lens, block=1)
    assert np.all(dq == 0) and np.all(dk == 0)
    assert max_abs(dv, np.asarray(case.dout, np.float64)) < 1e-15
    # GDPA with one-row blocks: O_i = act(S_ii) V_i (the block has one key: weight 1)
    g = custom_case(lens, lens, 1, 8, dtype="f32", mode="silu", seed=33)
    og, _ = oracle_mod.forward(g.q, g.k, g.v, lens, lens, mode="silu", block=1)
    q = np.asarray(g.q, np.float64)[:, 0]
    k = np.asarray(g.k, np.float64)[:, 0]
    s = (q * k).sum(-1) / math.sqrt(8)
    a = s / (1 + np.exp(-s))
    assert max_abs(og[:, 0], a[:, None] * np.asarray(g.v, np.float64)[:, 0]) < 1e-14


# ------------------------------------------------------------ bias gradient

def _torch_bias_grad(case, lens_q, lens_kv, bias, bias_kind, mode, causal, bucket_fn):
    """d<O, dO>/d bias by torch fp64 autograd, with the bias as the leaf (per-sample SDPA or the
    plain GDPA formula, as in the other pins)."""
    from tests.helpers import bias_matrix, gdpa_sample, sdpa_sample, visible_mask
    q = torch.as_tensor(np.asarray(case.q, np.float64))
    k = torch.as_tensor(np.asarray(case.k, np.float64))
    v = torch.as_tensor(np.asarray(case.v, np.float64))
    do = torch.as_tensor(np.asarray(case.dout, np.float64))
    leaf = torch.as_tensor(np.asarray(bias, np.float64)).clone().requires_grad_(True)
    H, d = q.shape[1], q.shape[2]
    scale = 1.0 / math.sqrt(d)
    loss = torch.zeros((), dtype=torch.float64)
    qo = ko = 0
    for b, (n, m) in enumerate(zip(lens_q, lens_kv)):
        n, m = int(n), int(m)
        for h in range(H):
            if n == 0 or m == 0:
                continue
            vis = visible_mask(n, m, causal)
            bmat = bias_matrix(leaf, bias_kind, h, n, m, H, b, lens_q, lens_kv, bucket_fn)
            qs, ks, vs = q[qo:qo + n, h], k[ko:ko + m, h], v[ko:ko + m, h]
            if mode == "softmax":
                o, _ = sdpa_sample(qs, ks, vs, bmat, vis, scale)
                dead = ~vis.any(dim=1)
                o = torch.where(dead[:, None], torch.zeros_like(o), o)
            else:
                o = gdpa_sample(qs, ks, vs, bmat, vis, scale, mode)
            loss = loss + (o * do[qo:qo + n, h]).sum()
        qo += n
        ko += m
    (g,) = torch.autograd.grad(loss, (leaf,))
    return g.numpy()


@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bias_kind", ["relpos", "dense"])
def test_bias_grad_vs_torch(oracle_mod, mode, causal, bias_kind):
    ql, kl = ([5, 0, 9, 12], [5, 0, 9, 12]) if causal else ([4, 7, 3], [9, 2, 3])
    case = custom_case(ql, kl, 2, 8, dtype="f32", mode=mode, causal=causal,
                       bias_kind=bias_kind, num_buckets=64, seed=71, bias_std=0.5)
    got = oracle_mod.bias_grad(case.q, case.k, case.v, case.dout, ql, kl, mode=mode,
                               causal=causal, bias=case.bias, bias_kind=bias_kind)
    want = _torch_bias_grad(case, ql, kl, case.bias, bias_kind, mode, causal,
                            oracle_mod.relpos_bucket)
    assert got.shape == want.shape
    assert max_abs(got, want) < 1e-11
    assert np.abs(want).max() > 1e-3          # the gradient is not trivially zero


def test_bias_grad_softmax_rows_sum_to_zero(oracle_mod):
    # softmax: sum_j dS_ij = sum_j P_ij (dP_ij - D_i) = D_i - D_i = 0 for every query row, so
    # every head's table gradient sums to zero over the buckets, and a dense bias's gradient
    # sums to zero along every row
    ql = [40, 17, 1, 60]
    case = custom_case(ql, ql, 3, 16, dtype="f32", mode="softmax", causal=True,
                       bias_kind="relpos", seed=72, bias_std=0.5)
    g = oracle_mod.bias_grad(case.q, case.k, case.v, case.dout, ql, ql, causal=True,
                             bias=case.bias)
    assert np.abs(g.sum(axis=1)).max() < 1e-12 * max(1.0, np.abs(g).max())
    dense = custom_case(ql, ql, 2, 16, dtype="f32", mode="softmax", causal=True,
                        bias_kind="dense", seed=73, bias_std=0.5)
    gd = oracle_mod.bias_grad(dense.q, dense.k, dense.v, dense.dout, ql, ql, causal=True,
                              bias=dense.bias, bias_kind="dense")
    off = 0
    for n in ql:
        blk = gd[off:off + 2 * n * n].reshape(2, n, n)
        assert np.abs(blk.sum(axis=2)).max() < 1e-12
        off += 2 * n * n


def test_bias_grad_block_attention_is_sum_over_blocks(oracle_mod):
    # the table is shared by all blocks: BlockAttention's table gradient equals that of every
    # block taken as a sample of its own, summed
    lens, w = [11, 0, 4, 9], 4
    case = custom_case(lens, lens, 2, 8, dtype="f32", mode="gelu", causal=True,
                       bias_kind="relpos", seed=74, bias_std=0.5)
    got = oracle_mod.bias_grad(case.q, case.k, case.v, case.dout, lens, lens, mode="gelu",
                               causal=True, bias=case.bias, block=w)
    blocks = _split_lengths(lens, w)
    want = _torch_bias_grad(case, blocks, blocks, case.bias, "relpos", "gelu", True,
                            oracle_mod.relpos_bucket)
    assert max_abs(got, want) < 1e-11


# ------------------------------------------------- fused normalisation + quantisation (row F4)

def test_rmsnorm_closed_forms(oracle_mod):
    """RMS normalisation against values worked by hand: a group [3, 4, 0, ...] of 32 has mean
    square 25/32, so y = x * sqrt(32/25); a constant group c gives c / sqrt(c^2 + eps)."""
    x = np.zeros((1, 32))
    x[0, :2] = [3.0, 4.0]
    y = oracle_mod.rmsnorm(x, eps=0.0)
    assert np.allclose(y[0, :2], [3.0 * np.sqrt(32 / 25), 4.0 * np.sqrt(32 / 25)], rtol=1e-15)
    assert np.all(y[0, 2:] == 0)
    c = np.full((1, 64), -2.5)
    y = oracle_mod.rmsnorm(c, eps=0.75)
    assert np.allclose(y, -2.5 / np.sqrt(6.25 + 0.75), rtol=1e-15)
    # the gain multiplies channel by channel (not transposed, not per group)
    w = np.arange(1, 65, dtype=np.float64)
    assert np.allclose(oracle_mod.rmsnorm(c, w, eps=0.75), -2.5 / np.sqrt(7.0) * w, rtol=1e-15)


def test_rmsnorm_invariants(oracle_mod):
    """Unit mean square per group (eps = 0, unit gain), invariance to a positive scale of the
    group, groups of n inside a longer last dimension normalised on their own."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 3, 128))
    y = oracle_mod.rmsnorm(x, eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    assert np.allclose(oracle_mod.rmsnorm(7.5 * x, eps=0.0), y, rtol=1e-13)
    x2 = x.copy()
    x2[..., 64:] *= 100.0                       # groups of 64: the second half scales alone
    y64 = oracle_mod.rmsnorm(x2, n=64, eps=0.0)
    assert np.allclose(y64[..., :64], oracle_mod.rmsnorm(x[..., :64], eps=0.0), rtol=1e-13)
    assert np.allclose(y64[..., 64:], oracle_mod.rmsnorm(x[..., 64:], eps=0.0), rtol=1e-13)


# ------------------------------------------------ operand-rounding magnitudes

@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal,bias_kind", [(False, "none"), (True, "relpos"), (False, "dense")])
def test_abs_terms_bound_outputs(oracle_mod, mode, causal, bias_kind):
    """Triangle inequality: every term is at least the magnitude of the output it bounds."""
    ql, kl = ([5, 0, 9, 1, 12], [5, 0, 9, 1, 12]) if causal else ([4, 7, 3, 6], [9, 2, 3, 1])
    case = custom_case(ql, kl, 2, 16, dtype="f32", mode=mode, causal=causal,
                       bias_kind=bias_kind, seed=140, bias_std=0.5)
    c = oracle_mod.case_abs_terms(case)
    o, _ = oracle_mod.case_forward(case)
    dq, dk, dv = oracle_mod.case_backward(case)
    for name, x in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert np.all(c[name] >= np.abs(x) * (1 - 1e-12) - 1e-300), name
    # a term is zero exactly where nothing is visible: the empty sample's rows
    assert np.all(c["O"][5:5] == 0)


def test_abs_terms_equal_outputs_when_signs_agree(oracle_mod):
    """Where no cancellation is possible the term equals the output's magnitude: softmax with
    V >= 0 (P >= 0) gives cO = O, with dO >= 0 gives cdV = dV; one key per sample gives
    |dQ| = cdQ (a single term), one query per sample gives |dK| = cdK, and GDPA with one key
    gives |O| = cO."""
    case = custom_case([6, 3, 8], [4, 9, 5], 2, 16, dtype="f32", mode="softmax",
                       bias_kind="dense", seed=141, bias_std=0.5)
    case.v = case.v.abs()
    case.dout = case.dout.abs()
    c = oracle_mod.case_abs_terms(case)
    o, _ = oracle_mod.case_forward(case)
    _, _, dv = oracle_mod.case_backward(case)
    assert max_abs(c["O"], o) < 1e-12 and max_abs(c["dV"], dv) < 1e-12
    for mode in ("softmax", "silu", "gelu"):
        one_k = custom_case([5, 3, 7], [1, 1, 1], 2, 16, dtype="f32", mode=mode,
                            bias_kind="relpos", seed=142, bias_std=0.5)
        c = oracle_mod.case_abs_terms(one_k)
        dq, _, _ = oracle_mod.case_backward(one_k)
        assert max_abs(c["dQ"], np.abs(dq)) < 1e-12, mode
        if mode != "softmax":
            o, _ = oracle_mod.case_forward(one_k)
            assert max_abs(c["O"], np.abs(o)) < 1e-12, mode
        one_q = custom_case([1, 1, 1], [5, 3, 7], 2, 16, dtype="f32", mode=mode,
                            bias_kind="dense", seed=143, bias_std=0.5)
        c = oracle_mod.case_abs_terms(one_q)
        _, dk, _ = oracle_mod.case_backward(one_q)
        assert max_abs(c["dK"], np.abs(dk)) < 1e-12, mode


def test_abs_terms_scale_with_operands(oracle_mod):
    """cO is linear in |V| and cdV in |dO| at fixed P; cdQ and cdK depend on V and dO only
    through dS (scaling V by 4 and dO by 1/4, both exact, leaves dP, dS and P unchanged)."""
    case = custom_case([6, 3], [4, 9], 2, 16, dtype="f32", mode="silu", seed=144)
    c1 = oracle_mod.case_abs_terms(case)
    case.v = case.v * 4.0
    case.dout = case.dout / 4.0
    c2 = oracle_mod.case_abs_terms(case)
    assert rel_l2(c2["O"], 4.0 * c1["O"]) < 1e-12
    assert rel_l2(c2["dQ"], c1["dQ"]) < 1e-12 and rel_l2(c2["dK"], c1["dK"]) < 1e-12
    assert rel_l2(c2["dV"], c1["dV"] / 4.0) < 1e-12


# ------------------------------------------------------------ sliding window

WINDOW_CASES = [
    # q_lens, kv_lens, H, d, window
    ([9, 0, 13, 1, 20], [9, 0, 13, 1, 20], 2, 8, 3),
    ([4, 11, 6], [9, 5, 6], 2, 8, 2),          # asymmetric: aligned position i + (m - n)
    ([7, 16], [7, 16], 1, 8, 1),
    ([12], [5], 1, 8, 7),
]


@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bias_kind", ["none", "relpos", "dense"])
@pytest.mark.parametrize("ci", range(len(WINDOW_CASES)))
def test_window_vs_torch(oracle_mod, mode, causal, bias_kind, ci):
    """Sliding window against torch fp64 SDPA / autograd with a band mask."""
    ql, kl, H, d, W = WINDOW_CASES[ci]
    case = custom_case(ql, kl, H, d, dtype="f32", mode=mode, causal=causal,
                       bias_kind=bias_kind, seed=150 + ci, bias_std=0.5)
    o, lse = oracle_mod.case_forward(case, window=W)
    dq, dk, dv = oracle_mod.case_backward(case, window=W)
    ref = torch_reference(case.q, case.k, case.v, case.q_lens, case.kv_lens, mode, causal,
                          case.bias, bias_kind, oracle_mod.relpos_bucket, dout=case.dout,
                          window=W)
    assert max_abs(o, ref["o"]) < 1e-12
    if mode == "softmax":
        finite = np.isfinite(ref["lse"])
        assert np.array_equal(np.isfinite(lse), finite)
        assert max_abs(lse[finite], ref["lse"][finite]) < 1e-12
    for got, want in ((dq, ref["dq"]), (dk, ref["dk"]), (dv, ref["dv"])):
        assert max_abs(got, want) < 1e-11


def test_window_special_cases(oracle_mod):
    """A window no shorter than every sample changes nothing (bit-identical); a causal window of
    one key gives softmax O_i = V_(i + m - n) (0 where that key does not exist), dQ = dK = 0 and
    dV_j = dO_(j - m + n); GDPA O_i = w act(S_i,i+m-n) V_(i+m-n)."""
    ql, kl = [9, 14, 3], [9, 10, 5]
    for mode in ("softmax", "gelu"):
        for causal in (False, True):
            case = custom_case(ql, kl, 2, 8, dtype="f32", mode=mode, causal=causal,
                               bias_kind="relpos", seed=160, bias_std=0.5)
            o0, l0 = oracle_mod.case_forward(case)
            o1, l1 = oracle_mod.case_forward(case, window=100)
            assert np.array_equal(o0, o1)
            g0 = oracle_mod.case_backward(case)
            g1 = oracle_mod.case_backward(case, window=100)
            assert all(np.array_equal(a, b) for a, b in zip(g0, g1))
    case = custom_case(ql, kl, 2, 8, dtype="f32", mode="softmax", causal=True, seed=161)
    o, lse = oracle_mod.case_forward(case, window=1)
    dq, dk, dv = oracle_mod.case_backward(case, window=1)
    v, do = case.v.double().numpy(), case.dout.double().numpy()
    qo, ko = 0, 0
    want_o = np.zeros_like(o)
    want_dv = np.zeros_like(dv)
    for n, m in zip(ql, kl):
        for i in range(n):
            j = i + m - n
            if 0 <= j < m:
                want_o[qo + i] = v[ko + j]
                want_dv[ko + j] = do[qo + i]
        qo += n
        ko += m
    assert max_abs(o, want_o) < 1e-15 and max_abs(dv, want_dv) < 1e-15
    assert np.all(dq == 0) and np.all(dk == 0)
    # rows whose only key would lie before the sample (i + m - n < 0) see nothing
    assert lse[0, 9 + 0] == -np.inf and np.all(o[9:13] == 0)


def _vis_w(n, m, causal, W, i, j):
    d = i + (m - n) - j
    return (not causal or d >= 0) and (W == 0 or abs(d) < W)


def _pairs_w(n, m, causal, W, r0, r1, c0, c1):
    return sum(1 for i in range(max(r0, 0), min(r1, n)) for j in range(max(c0, 0), min(c1, m))
               if _vis_w(n, m, causal, W, i, j))


@pytest.mark.parametrize("seed", range(8))
def test_schedule_window_bruteforce(oracle_mod, seed):
    """With a window every list entry covers exactly the steps its tile can see: its first and
    last steps hold a visible pair, the steps outside its range hold none (forward, both
    backward lists); chunks of a split tile still tile the range; order stays longest first."""
    rng = np.random.default_rng(300 + seed)
    B = int(rng.integers(1, 9))
    ql = rng.integers(0, 400, size=B).astype(np.int32)
    kl = ql.copy() if seed % 2 == 0 else rng.integers(0, 400, size=B).astype(np.int32)
    causal = seed % 3 != 1
    W = int(rng.choice([1, 5, 40, 64, 100, 333]))
    bm, bn = 64 * int(rng.integers(1, 3)), 64
    slots = int(rng.integers(1, 30)) if seed % 4 else 0
    qo, ko = oracle_mod.offsets(ql), oracle_mod.offsets(kl)
    s = oracle_mod.schedule(qo, ko, 2, causal, bm=bm, bn=bn, slots=slots, bq_bm=64, bq_bn=64,
                            bk_bn=128, bk_bm=64, fuse=0, window=W)
    fwd = s["fwd"]
    cost = np.maximum(1, fwd[:, 3] - fwd[:, 2])
    keys = [(-c, b, t, kb) for c, (b, t, kb, _) in zip(cost, fwd)]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)

    def check_range(n, m, rows, lo, hi, step, along_keys):
        # [lo, hi) steps of `step` rows along keys (or queries) for the row (column) block rows
        r0, r1 = rows
        def cnt(a, b):
            return _pairs_w(n, m, causal, W, r0, r1, a, b) if along_keys else \
                _pairs_w(n, m, causal, W, a, b, r0, r1)
        total = cnt(0, 1 << 30)
        if hi > lo:
            assert cnt(lo * step, hi * step) == total
            assert cnt(lo * step, (lo + 1) * step) > 0 and cnt((hi - 1) * step, hi * step) > 0
        else:
            assert total == 0

    for b in range(B):
        n, m = int(ql[b]), int(kl[b])
        for t in range(-(-n // bm)):
            parts = sorted([tuple(r[2:]) for r in fwd if r[0] == b and r[1] == t])
            for a, c in zip(parts, parts[1:]):
                assert a[1] == c[0]
            check_range(n, m, (t * bm, (t + 1) * bm), parts[0][0], parts[-1][1], bn, True)
        for _, t, lo, hi in (r for r in s["bwd_q"] if r[0] == b):
            check_range(n, m, (t * 64, (t + 1) * 64), lo, hi, 64, True)
        for _, u, lo, hi in (r for r in s["bwd_kv"] if r[0] == b):
            check_range(n, m, (u * 128, (u + 1) * 128), lo, hi, 64, False)
