"""GPU parity of the decode over an FP8 K/V cache (attn_fp8_decode) against the
oracle (oracle.decode) on the same seeded inputs.

The cache and the new queries are quantised by quantize_qkv_fp8 on the GPU
(checked bit-exact against the oracle's quantiser), and the oracle runs its
own quantiser on the same float inputs.  O and LSE are held to the dense
path's contract: E1, the exact attention of the dequantised queries against
the dequantised cache (no split), within RMSE 2e-3 and max-abs 2e-2 widened
only by the bars derived from E1 (tests.gpu_common.check_fp8_vs_e1).  The
kernel-shaped loop with the kernel's split is printed as a diagnostic.
"""

import numpy as np
import pytest
import torch

import fp8_attention_forward_amd as fa
import workloads
from oracle import decode as od
from oracle import quantize as oq
from tests.gpu_common import check_fp8_vs_e1, dev, host, rms

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

CASES = [
    # B, Hq, Hkv, Sq, Ncap, D, scale_block, hadamard, causal, seqlens, split, kind
    (2, 8, 2, 1, 1000, 128, 128, True, True, [1000, 333], 64, "outlier"),
    (3, 4, 4, 2, 700, 64, 64, True, True, [700, 2, 65], 128, "iid"),
    (1, 32, 4, 4, 2048, 128, 128, True, False, [2048], 0, "iid"),
    (2, 2, 1, 3, 513, 128, 64, False, True, [513, 300], 64, "outlier"),
    (1, 8, 8, 1, 5000, 128, 128, True, True, [4097], 256, "iid"),
    (2, 16, 2, 4, 3000, 64, 128, True, True, [2999, 64], 0, "outlier"),
    (1, 1, 1, 1, 64, 128, 64, True, False, [1], 64, "iid"),
    (1, 1, 1, 1, 64, 128, 64, True, False, [1], 0, "iid"),
    # balanced shares (split 0): many short sequences, shares that cross
    # (sequence, K/V head) segments, more than 64 sequences (several per lane
    # of the length scan), more waves than tiles, lengths at Sq and at Ncap
    (64, 4, 2, 1, 4096, 128, 128, True, True, ("rand", 1, 640), 0, "iid"),
    (200, 2, 2, 2, 2048, 64, 64, True, True, ("rand", 2, 641), 0, "outlier"),
    (300, 2, 1, 1, 256, 128, 128, False, False, ("rand", 1, 642), 0, "iid"),
    # above the balanced schedule's batch limit: fixed ranges
    (520, 1, 1, 1, 128, 64, 64, True, True, ("rand", 1, 643), 0, "iid"),
]
IDS = ["B{}Hq{}Hkv{}Sq{}N{}D{}sb{}had{}c{}s{}".format(*(int(x) if isinstance(x, bool) else x
                                                        for x in c[:9] + (c[10],))) for c in CASES]


def _seqlens(spec, B, Ncap):
    if isinstance(spec, tuple):                   # ("rand", lowest length, seed), the ends included
        _, lo, seed = spec
        L = np.random.default_rng(seed).integers(lo, Ncap + 1, size=B)
        L[0], L[-1] = lo, Ncap
        return L.astype(np.int32)
    return np.asarray(spec, dtype=np.int32)


def _run(case, seed_off=0):
    B, Hq, Hkv, Sq, Ncap, D, sb, had, causal, seqlens, split, kind = case
    q, k, v = workloads.generate_decode(kind, B, Hq, Hkv, Sq, Ncap, D, 60 + Ncap + seed_off)
    seqlens = _seqlens(seqlens, B, Ncap)
    print(f"\n[decode] {case[:9]} seqlens {seqlens.tolist()} split {split}", flush=True)
    # the cache: the sequences' K and V quantised as one call would (Q slot unused)
    _, k8, v8, _, kd, vd = fa.quantize_qkv_fp8(dev(k), dev(k), dev(v), scale_block=sb, hadamard=had, seed=0x5EED)
    # the new queries: their own quantiser call (one block), same sign vector
    q8, _, _, qd, _, _ = fa.quantize_qkv_fp8(dev(q), dev(q), dev(q), scale_block=sb, hadamard=had, seed=0x5EED)
    o, lse = fa.attn_fp8_decode(q8, qd, k8, v8, kd, vd, dev(seqlens), scale_block=sb, hadamard=had,
                                causal=causal, split=split)
    torch.cuda.synchronize()
    # (the diagnostic split loop: the kernel's fixed ranges, or one range per
    # sequence for the balanced shares)
    used = fa.attn_fp8_decode_split(B, Hkv, Ncap, split) or -(-Ncap // 64) * 64
    ref_k = oq.quantize_qkv(k, k, v, sb, had, 0x5EED)
    ref_q = oq.quantize_qkv(q, q, q, sb, had, 0x5EED)
    for g, r, nm in ((k8, ref_k[1], "k8"), (v8, ref_k[2], "v8"), (q8, ref_q[0], "q8")):
        assert np.array_equal(host(g), r), f"{nm} codes differ"
    for g, r, nm in ((kd, ref_k[4], "kd"), (vd, ref_k[5], "vd"), (qd, ref_q[3], "qd")):
        assert np.array_equal(host(g).view(np.uint32), r.view(np.uint32)), f"{nm} descales differ"
    bars = od.emulated_fp8_decode_bars(ref_q[0], ref_q[3], ref_k[1], ref_k[2], ref_k[4], ref_k[5], seqlens, sb,
                                       had, causal)
    o2, _ = od.emulated_fp8_decode(ref_q[0], ref_q[3], ref_k[1], ref_k[2], ref_k[4], ref_k[5], seqlens, sb, had,
                                   causal, used)
    return host(o), host(lse), bars, o2, used


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_decode_matches_e1(case):
    o, lse, bars, o2, used = _run(case)
    check_fp8_vs_e1(o, lse, bars, tag=f"{case[:9]} split {used}")
    print(f"  split {used}: diagnostic RMSE vs the split loop {rms(o - o2):.3e}", flush=True)


def test_decode_run_to_run_bitwise():
    case = CASES[0]
    a = _run(case)
    b = _run(case)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_decode_with_one_range_is_the_dense_loop():
    # one range covering the whole sequence, Sq = L (every token a query, G = 1):
    # the same loop as attn_fp8_fwd, up to the V reference (equal here: one block)
    B, H, L, D, sb = 1, 2, 32, 128, 64
    q, k, v = workloads.generate_decode("iid", B, H, H, L, L, D, 9)
    qq = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=sb, seed=0x5EED)
    o_dense, l_dense = fa.attn_fp8_fwd(*qq, scale_block=sb, causal=True)
    o_dec, l_dec = fa.attn_fp8_decode(qq[0], qq[3], qq[1], qq[2], qq[4], qq[5], dev(np.array([L], np.int32)),
                                      scale_block=sb, causal=True, split=64)
    torch.cuda.synchronize()
    assert rms(host(o_dec) - host(o_dense)) <= 1e-3
    assert np.allclose(host(l_dec), host(l_dense), rtol=1e-5, atol=1e-5)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["decode_gqa", "decode_gqa_spec"])
def test_decode_workload_parity(name):
    w = workloads.DECODE_WORKLOADS[name]
    seqlens = w.seqlens()
    print(f"\n[{name}] generating B{w.B} Hq{w.Hq} Hkv{w.Hkv} Sq{w.Sq} Ncap{w.Ncap} D{w.D}", flush=True)
    q, k, v = workloads.generate_decode_workload(w)
    _, k8, v8, _, kd, vd = fa.quantize_qkv_fp8(dev(k), dev(k), dev(v), scale_block=w.scale_block,
                                               hadamard=w.hadamard, seed=w.sign_seed)
    q8, _, _, qd, _, _ = fa.quantize_qkv_fp8(dev(q), dev(q), dev(q), scale_block=w.scale_block,
                                             hadamard=w.hadamard, seed=w.sign_seed)
    o, lse = fa.attn_fp8_decode(q8, qd, k8, v8, kd, vd, dev(seqlens), scale_block=w.scale_block,
                                hadamard=w.hadamard, causal=w.causal)
    torch.cuda.synchronize()
    used = fa.attn_fp8_decode_split(w.B, w.Hkv, w.Ncap, 0)
    for b in sorted({0, int(np.argmax(seqlens)), int(np.argmin(seqlens))}):
        for hk in sorted({0, w.Hkv - 1}):
            G = w.Hq // w.Hkv
            hs = slice(hk * G, (hk + 1) * G)
            ref_k = oq.quantize_qkv(k[b:b + 1, hk:hk + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1],
                                    w.scale_block, w.hadamard, w.sign_seed)
            ref_q = oq.quantize_qkv(q[b:b + 1, hs], q[b:b + 1, hs], q[b:b + 1, hs], w.scale_block, w.hadamard,
                                    w.sign_seed)
            assert np.array_equal(host(k8[b:b + 1, hk:hk + 1]), ref_k[1])
            assert np.array_equal(host(v8[b:b + 1, hk:hk + 1]), ref_k[2])
            assert np.array_equal(host(q8[b:b + 1, hs]), ref_q[0])
            bars = od.emulated_fp8_decode_bars(ref_q[0], ref_q[3], ref_k[1], ref_k[2], ref_k[4], ref_k[5],
                                               seqlens[b:b + 1], w.scale_block, w.hadamard, w.causal)
            og, lg = host(o[b:b + 1, hs]), host(lse[b:b + 1, hs])
            check_fp8_vs_e1(og, lg, bars, tag=f"[{name}] b {b} (L {int(seqlens[b])}) kv head {hk}")
