"""Seeded random-shape sweeps of the three FP8 paths against the oracle (GPU).

Each case draws its shape and options from a fixed seed: sequence lengths
(ragged against the 64-key and 128-query tiles), head dimension, scale block,
rotation, causal mask, the MX options (block and 32-channel scales) and
Schraudolph's exponential, document lengths
(packed path) and cache lengths, grouping and new-token counts (decode).
The bars are those of the fixed-shape tests: quantiser bit-exact, O / LSE
against E1 (the exact attention of the quantised inputs) within RMSE 2e-3 and
max-abs 2e-2, widened only by the bars derived from E1 for P's e4m3 rounding,
the matrix cores' accumulation (pinned in test_gpu_numerics) and the
Schraudolph option; rotated and unrotated cases alike.
"""

import numpy as np
import pytest
import torch

import fp8_attention_forward_amd as fa
import workloads
from oracle import attention as oatt
from oracle import decode as odec
from oracle import quantize as oq
from oracle import varlen as ov
from tests.gpu_common import check_fp8_vs_e1, dev, host, rms

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _draw(seed):
    rng = np.random.default_rng(seed)
    return rng, dict(D=int(rng.choice([64, 128])), sb=int(rng.choice([64, 128])), had=bool(rng.random() < 0.8),
                     causal=bool(rng.random() < 0.5), mx=bool(rng.random() < 0.3),
                     exp2="schraudolph" if rng.random() < 0.3 else "exact")


def _mx32(seed):
    # (drawn from a stream of its own, so the other draws of a seed stay as they were)
    return bool(np.random.default_rng(seed + 7919).random() < 0.3)


@pytest.mark.parametrize("seed", range(16))
def test_dense_sweep(seed):
    rng, c = _draw(1000 + seed)
    B, H, N = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 900))
    m32 = _mx32(seed)
    if m32:
        c["mx"] = False
    print(f"\n[dense sweep {seed}] B{B} H{H} N{N} {c} mx32={m32}", flush=True)
    q, k, v = workloads.generate("outlier", B, H, N, c["D"], 5000 + seed)
    qq = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=c["sb"], hadamard=c["had"], mx=c["mx"], mx32=m32)
    o, lse = fa.attn_fp8_fwd(*qq, scale_block=c["sb"], hadamard=c["had"], causal=c["causal"], exp2=c["exp2"],
                             mx=c["mx"], mx32=m32)
    torch.cuda.synchronize()
    ref = oq.quantize_qkv(q, k, v, c["sb"], c["had"], 0x5EED, pow2=c["mx"] or m32, group=32 if m32 else None)
    for g, r in zip(qq, ref):
        g = host(g)
        assert np.array_equal(g if r.dtype == np.uint8 else g.view(np.uint32),
                              r if r.dtype == np.uint8 else r.view(np.uint32))
    bars = oatt.emulated_fp8_attention_bars(*ref, c["sb"], c["had"], c["causal"], exp2=c["exp2"])
    check_fp8_vs_e1(host(o), host(lse), bars, tag=f"dense sweep {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_packed_sweep(seed):
    rng, c = _draw(2000 + seed)
    H = int(rng.integers(1, 4))
    lens = rng.integers(0, 400, size=int(rng.integers(1, 12)))
    lens[rng.integers(0, len(lens))] = max(1, int(lens.max()))    # at least one token
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    print(f"\n[packed sweep {seed}] H{H} T{T} docs {lens.tolist()} {c}", flush=True)
    q, k, v = workloads.generate_packed("outlier", H, T, c["D"], 6000 + seed)
    cu_d = dev(cu)
    qq = fa.quantize_qkv_fp8_varlen(dev(q), dev(k), dev(v), cu_d, scale_block=c["sb"], hadamard=c["had"],
                                    mx=c["mx"])
    o, lse = fa.attn_fp8_fwd_varlen(*qq, cu_d, scale_block=c["sb"], hadamard=c["had"], causal=c["causal"],
                                    exp2=c["exp2"], mx=c["mx"])
    torch.cuda.synchronize()
    ref = ov.quantize_qkv_varlen(q, k, v, cu, c["sb"], c["had"], 0x5EED, pow2=c["mx"])
    for g, r in zip(qq[:3], ref[:3]):
        assert np.array_equal(host(g), r)
    for g, r in zip(qq[3:], ref[3:]):
        used = ~np.isnan(r)
        assert np.array_equal(host(g)[used].view(np.uint32), r[used].view(np.uint32))
    bars = ov.emulated_fp8_attention_varlen_bars(*ref, cu, c["sb"], c["had"], c["causal"], exp2=c["exp2"])
    check_fp8_vs_e1(host(o), host(lse), bars, tag=f"packed sweep {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_decode_sweep(seed):
    rng, c = _draw(3000 + seed)
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    Sq = int(rng.choice([1, 2, 4]))
    while G * Sq > 32:
        Sq //= 2
    B = int(rng.integers(1, 4))
    N = int(rng.integers(Sq, 3000))
    seqlens = rng.integers(Sq, N + 1, size=B).astype(np.int32)
    split = int(rng.choice([0, 64, 192, 512]))
    print(f"\n[decode sweep {seed}] B{B} Hq{Hkv * G} Hkv{Hkv} Sq{Sq} N{N} lens {seqlens.tolist()} split {split} "
          f"D{c['D']} sb{c['sb']} had{c['had']} causal{c['causal']}", flush=True)
    q, k, v = workloads.generate_decode("outlier", B, Hkv * G, Hkv, Sq, N, c["D"], 7000 + seed)
    _, k8, v8, _, kd, vd = fa.quantize_qkv_fp8(dev(k), dev(k), dev(v), scale_block=c["sb"], hadamard=c["had"])
    q8, _, _, qd, _, _ = fa.quantize_qkv_fp8(dev(q), dev(q), dev(q), scale_block=c["sb"], hadamard=c["had"])
    o, lse = fa.attn_fp8_decode(q8, qd, k8, v8, kd, vd, dev(seqlens), scale_block=c["sb"], hadamard=c["had"],
                                causal=c["causal"], split=split)
    torch.cuda.synchronize()
    rk = oq.quantize_qkv(k, k, v, c["sb"], c["had"], 0x5EED)
    rq = oq.quantize_qkv(q, q, q, c["sb"], c["had"], 0x5EED)
    bars = odec.emulated_fp8_decode_bars(rq[0], rq[3], rk[1], rk[2], rk[4], rk[5], seqlens, c["sb"], c["had"],
                                         c["causal"])
    check_fp8_vs_e1(host(o), host(lse), bars, tag=f"decode sweep {seed}")
