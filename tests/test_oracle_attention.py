"""Pins of the oracle's attention: brute force, the running-softmax loop of the
sketch, closed forms, and invariance under the orthogonal rotation."""

import itertools
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import attention, e4m3, quantize
from oracle.philox import sign_vector


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("n,d", [(1, 4), (3, 4), (6, 8), (5, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(n, d, causal):
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    scale = 1 / math.sqrt(d)
    o, lse = attention.attention_fp64(q, k, v, causal, scale)
    ob, lb = attention.brute_force_attention(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    assert np.allclose(o, ob, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lb, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("block_c", [1, 3, 64, 128, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_equals_two_pass(block_c, causal):
    n, d = 200, 32
    q, k, v = _rand((n, d), 4, 2.0), _rand((n, d), 5, 2.0), _rand((n, d), 6)
    scale = 1 / math.sqrt(d)
    o, lse = attention.attention_fp64(q, k, v, causal, scale, row_chunk=37)
    oo, lo = attention.online_attention_fp64(q, k, v, causal, scale, block_c)
    assert np.allclose(o, oo, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lo, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_uniform_weights(causal):
    n, d = 50, 16
    q = np.zeros((n, d))
    k, v = _rand((n, d), 7), _rand((n, d), 8)
    o, lse = attention.reference_attention(q, k, v, causal)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    assert np.allclose(lse, np.log(cnt), rtol=0, atol=1e-14)
    means = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.tile(v.mean(axis=0), (n, 1))
    assert np.allclose(o, means, rtol=0, atol=1e-13)


def test_constant_values_pass_through():
    n, d = 40, 8
    q, k = _rand((n, d), 9, 3.0), _rand((n, d), 10, 3.0)
    c = _rand((d,), 11)
    v = np.tile(c, (n, 1))
    for causal in (False, True):
        o, _ = attention.reference_attention(q, k, v, causal)
        assert np.allclose(o, np.tile(c, (n, 1)), rtol=0, atol=1e-13)


def test_causal_first_row():
    n, d = 30, 8
    q, k, v = _rand((n, d), 12), _rand((n, d), 13), _rand((n, d), 14)
    o, lse = attention.reference_attention(q, k, v, True)
    assert np.array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(q[0] @ k[0] / math.sqrt(d), abs=1e-14)


def test_dominant_key_selects_its_value():
    n, d = 20, 4
    k = np.eye(n, d) * 0
    k[:, 0] = np.arange(n)                       # key j scores proportional to j
    q = np.zeros((n, d))
    q[:, 0] = 60.0 * math.sqrt(d)                # margin between keys >= 60
    v = _rand((n, d), 15)
    o, lse = attention.reference_attention(q, k, v, False)
    assert np.allclose(o, np.tile(v[-1], (n, 1)), atol=1e-20 + math.exp(-50) * np.abs(v).max())
    assert np.allclose(lse, 60.0 * (n - 1), rtol=1e-15)


def test_rotation_invariance_all_signs_d4():
    n, d = 12, 4
    q, k, v = _rand((n, d), 16), _rand((n, d), 17), _rand((n, d), 18)
    h = scipy.linalg.hadamard(d).astype(np.float64)
    o0, l0 = attention.reference_attention(q, k, v, True)
    for signs in itertools.product([-1.0, 1.0], repeat=d):
        s = np.array(signs)
        rq, rk = (q * s) @ h, (k * s) @ h
        o, l = attention.attention_fp64(rq, rk, v, True, 1 / (math.sqrt(d) * d))
        assert np.allclose(o, o0, rtol=1e-12, atol=1e-13)
        assert np.allclose(l, l0, rtol=1e-12, atol=1e-13)


def test_rows_subset_matches_full():
    q, k, v = _rand((2, 3, 100, 16), 19), _rand((2, 3, 100, 16), 20), _rand((2, 3, 100, 16), 21)
    o, l = attention.reference_attention(q, k, v, True)
    rows = [0, 5, 63, 99]
    os_, ls = attention.reference_attention(q, k, v, True, rows=rows)
    assert np.array_equal(o[..., rows, :], os_) and np.array_equal(l[..., rows], ls)


def _grid_inputs(shape, seed):
    """Values that block quantisation reproduces exactly: e4m3 values times 2^k,
    with every block containing +-448 * 2^k."""
    from oracle import e4m3
    rng = np.random.default_rng(seed)
    codes = rng.choice(e4m3.all_finite_codes(), size=shape)
    x = e4m3.decode(codes)
    x[..., ::64, 0] = 448.0
    return (x * 2.0 ** -6).astype(np.float32)


def test_emulated_attention_is_reference_on_exact_inputs():
    shape = (1, 2, 128, 64)
    q, k, v = (_grid_inputs(shape, s) for s in (22, 23, 24))
    q8, k8, v8, qd, kd, vd = quantize.quantize_qkv(q, k, v, 64, False, 0)
    for causal in (False, True):
        oe, le = attention.emulated_fp8_attention(q8, k8, v8, qd, kd, vd, 64, False, causal)
        orf, lr = attention.reference_attention(q, k, v, causal)
        assert np.array_equal(oe, orf) and np.array_equal(le, lr)


def test_emulated_attention_with_rotation_tracks_reference():
    shape = (1, 2, 256, 64)
    q, k, v = (_rand(shape, s).astype(np.float32) for s in (25, 26, 27))
    q8, k8, v8, qd, kd, vd = quantize.quantize_qkv(q, k, v, 64, True, 0x5EED)
    oe, le = attention.emulated_fp8_attention(q8, k8, v8, qd, kd, vd, 64, True, False)
    orf, lr = attention.reference_attention(q, k, v, False)
    rel = np.sqrt(np.mean((oe - orf) ** 2)) / np.sqrt(np.mean(orf ** 2))
    assert rel < 0.08                           # e4m3 carries ~2^-4 relative error
    assert np.max(np.abs(le - lr)) < 0.1
    # a dropped 1/d would scale scores by 64: the LSE would be far off
    o_bad, l_bad = attention.attention_fp64(quantize.dequantize(q8, qd, 64), quantize.dequantize(k8, kd, 64),
                                            quantize.dequantize(v8, vd, 64), False, 1 / math.sqrt(64))
    assert np.max(np.abs(l_bad - lr)) > 1.0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tau", [0.0, 8.0])
@pytest.mark.parametrize("had", [False, True])
def test_tiled_fp8_loop_without_p_rounding_equals_e1(causal, tau, had):
    shape = (1, 2, 300, 64)
    q, k, v = (_rand(shape, s, 2.0).astype(np.float32) for s in (28, 29, 30))
    v[0, 1, 128:192] *= 0.05                  # a V block with a much smaller scale
    qq = quantize.quantize_qkv(q, k, v, 64, had, 0x5EED)
    o1, l1 = attention.emulated_fp8_attention(*qq, 64, had, causal)
    o2, l2 = attention.emulated_fp8_attention_tiled(*qq, 64, had, causal, tau=tau, quantize_p=False,
                                                     bf16_output=False)
    assert np.allclose(o2, o1, rtol=1e-11, atol=1e-13)
    assert np.allclose(l2, l1, rtol=1e-12, atol=1e-13)
    # rounding P moves O by e4m3's relative step at most, and never the LSE
    o3, l3 = attention.emulated_fp8_attention_tiled(*qq, 64, had, causal, tau=tau, bf16_output=False)
    assert np.allclose(l3, l1, rtol=1e-12, atol=1e-13)
    vmax = np.abs(quantize.dequantize(qq[2], qq[5], 64)).max()
    assert np.max(np.abs(o3 - o1)) <= 2.0 ** -4 * vmax
    assert not np.array_equal(o3, o1)


def test_tiled_fp8_loop_rows_subset():
    shape = (1, 1, 200, 64)
    q, k, v = (_rand(shape, s).astype(np.float32) for s in (31, 32, 33))
    qq = quantize.quantize_qkv(q, k, v, 64, True, 1)
    o, l = attention.emulated_fp8_attention_tiled(*qq, 64, True, True)
    rows = [0, 63, 64, 199]
    o2, l2 = attention.emulated_fp8_attention_tiled(*qq, 64, True, True, rows=rows)
    assert np.array_equal(o[..., rows, :], o2) and np.array_equal(l[..., rows], l2)


@pytest.mark.parametrize("tau,lift", [(0.0, 0.0), (0.0, 4.0), (8.0, 4.0), (2.0, 1.0)])
def test_tiled_fp8_loop_brute_force_tiny(tau, lift):
    # two key blocks of 2 keys, d = 4: explicit loops with the stated P rule
    # (the reference moves to lift below a block's max when that max exceeds
    # it by more than tau)
    from oracle import e4m3
    rng = np.random.default_rng(34)
    shape = (1, 1, 4, 4)
    q, k, v = (rng.standard_normal(shape).astype(np.float32) for _ in range(3))
    q[0, 0, 3] *= 8.0                      # a row whose second block moves the reference under every tau
    k[0, 0, 3] *= 8.0
    qq = quantize.quantize_qkv(q, k, v, 2, False, 0)
    q8, k8, v8, qd, kd, vd = qq
    o, lse = attention.emulated_fp8_attention_tiled(*qq, 2, False, False, tau=tau, lift=lift, bf16_output=False,
                                                     block_c=2)
    dq = e4m3.decode(q8)[0, 0]
    dk = e4m3.decode(k8)[0, 0]
    dv = e4m3.decode(v8)[0, 0]
    c = math.log2(math.e) / 2.0
    moved = 0
    for i in range(4):
        t = [sum(dq[i, x] * dk[j, x] for x in range(4)) * qd[0, 0, i // 2] * kd[0, 0, j // 2] * c for j in range(4)]
        m0 = max(t[0], t[1]) - lift
        m1 = max(t[2], t[3]) - lift if max(t[2], t[3]) > m0 + tau else m0
        moved += m1 != m0
        num = [0.0] * 4
        for j in range(4):
            mj = m0 if j < 2 else m1
            pj = float(e4m3.decode(e4m3.encode(2.0 ** (t[j] - mj))))
            w = 2.0 ** (mj - m1)
            for x in range(4):
                num[x] += w * pj * dv[j, x] * vd[0, 0, j // 2]
        l = sum(2.0 ** (tj - m1) for tj in t)
        for x in range(4):
            assert o[0, 0, i, x] == pytest.approx(num[x] / l, rel=1e-12, abs=1e-14)
        assert lse[0, 0, i] == pytest.approx(math.log(2) * (m1 + math.log2(l)), rel=1e-12)
    assert moved >= 1


def test_round_to_bf16_matches_torch():
    import torch
    rng = np.random.default_rng(35)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000),
                        [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -(1.0 + 2.0 ** -8)]])
    x = x.astype(np.float32).astype(np.float64)      # float32 values: one rounding on both sides
    ours = attention.round_to_bf16(x)
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    fin = np.abs(x) < 3e38
    assert np.array_equal(ours[fin], ref[fin])
    assert np.signbit(ours[-5]) and ours[-4] == 1.0
    assert ours[-3] == 1.0 and ours[-2] == 1.0 + 2.0 ** -7 and ours[-1] == -1.0   # ties to even


def test_tiled_fp8_loop_output_is_bf16_rounded():
    shape = (1, 1, 128, 64)
    q, k, v = (_rand(shape, s).astype(np.float32) for s in (36, 37, 38))
    qq = quantize.quantize_qkv(q, k, v, 64, True, 2)
    o_raw, l_raw = attention.emulated_fp8_attention_tiled(*qq, 64, True, False, bf16_output=False)
    o, l = attention.emulated_fp8_attention_tiled(*qq, 64, True, False)
    assert np.array_equal(o, attention.round_to_bf16(o_raw)) and np.array_equal(l, l_raw)


def test_tiled_fp8_loop_block_size_only_moves_p_rounding():
    shape = (1, 2, 300, 64)
    q, k, v = (_rand(shape, s).astype(np.float32) for s in (39, 40, 41))
    qq = quantize.quantize_qkv(q, k, v, 128, True, 3)
    o1, l1 = attention.emulated_fp8_attention(*qq, 128, True, True)
    kw = dict(quantize_p=False, bf16_output=False)
    for bc in (32, 64, 128):
        o, l = attention.emulated_fp8_attention_tiled(*qq, 128, True, True, block_c=bc, **kw)
        assert np.allclose(o, o1, rtol=1e-11, atol=1e-13) and np.allclose(l, l1, rtol=1e-12)
    with pytest.raises(ValueError):
        attention.emulated_fp8_attention_tiled(*qq, 128, True, True, block_c=48)


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_mx_loop_without_p_rounding_equals_e1(causal):
    # power-of-two scales applied to the operands: without P rounding the loop
    # is E1 on the same (pow2-quantised) inputs
    shape = (1, 2, 300, 64)
    q, k, v = (_rand(shape, s, 3.0).astype(np.float32) for s in (40, 41, 42))
    v[0, 1, 128:192] *= 0.01
    qq = quantize.quantize_qkv(q, k, v, 64, True, 0x5EED, pow2=True)
    o1, l1 = attention.emulated_fp8_attention(*qq, 64, True, causal)
    o2, l2 = attention.emulated_fp8_attention_tiled(*qq, 64, True, causal, quantize_p=False, bf16_output=False)
    assert np.allclose(o2, o1, rtol=1e-11, atol=1e-13)
    assert np.allclose(l2, l1, rtol=1e-12, atol=1e-13)


def test_tiled_mx_loop_brute_force_tiny():
    # two key blocks of 2 keys, d = 4, power-of-two scales for Q and K too:
    # P = e4m3(2^(t - m)), V's scale on V itself
    from oracle import e4m3
    rng = np.random.default_rng(43)
    shape = (1, 1, 4, 4)
    q, k, v = (rng.standard_normal(shape).astype(np.float32) for _ in range(3))
    v[0, 0, 2:] *= 0.1
    qq = quantize.quantize_qkv(q, k, v, 2, False, 0, pow2=True)
    q8, k8, v8, qd, kd, vd = qq
    o, lse = attention.emulated_fp8_attention_tiled(*qq, 2, False, False, tau=0.0, lift=0.0, bf16_output=False,
                                                     block_c=2)
    dq, dk, dv = (e4m3.decode(x)[0, 0] for x in (q8, k8, v8))
    c = math.log2(math.e) / 2.0
    for i in range(4):
        t = [sum(dq[i, x] * dk[j, x] for x in range(4)) * qd[0, 0, i // 2] * kd[0, 0, j // 2] * c for j in range(4)]
        m0 = max(t[0], t[1])
        m1 = max(m0, t[2], t[3])
        num = [0.0] * 4
        for j in range(4):
            mj = m0 if j < 2 else m1
            pj = float(e4m3.decode(e4m3.encode(2.0 ** (t[j] - mj))))
            for x in range(4):
                num[x] += 2.0 ** (mj - m1) * pj * dv[j, x] * vd[0, 0, j // 2]
        l = sum(2.0 ** (tj - m1) for tj in t)
        for x in range(4):
            assert o[0, 0, i, x] == pytest.approx(num[x] / l, rel=1e-12, abs=1e-14)
        assert lse[0, 0, i] == pytest.approx(math.log(2) * (m1 + math.log2(l)), rel=1e-12)


