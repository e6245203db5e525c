"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

* quantize_qkv_fp8: codes and descales bit-exact against the oracle's float32
  emulation (oracle.quantize).
* attn_fp8_fwd (and its options): O and LSE against E1, the exact float64
  attention of the dequantised inputs (oracle.emulated_fp8_attention): RMSE
  2e-3, max-abs 2e-2, LSE 2e-3 * max(1, |LSE|), each widened only by the bars
  that oracle.emulated_fp8_attention_bars derives from E1's own quantities
  for P's e4m3 rounding, the matrix cores' accumulation and (option)
  Schraudolph's exponential, plus half a BF16 ulp of the output.  The
  kernel-shaped loop E2 is printed as a diagnostic.
* attn_bf16_fwd: against exact FP64 attention of the BF16-rounded inputs.

Small shapes are checked in full; they span several tiles and a ragged tail.
"""

import math

import numpy as np
import pytest
import torch

import fp8_attention_forward_amd as fa
import workloads
from oracle import attention as oatt
from oracle import quantize as oq
from tests.gpu_common import bf16_round, check_fp8_vs_e1, dev, gpu_quantize, host, rms

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

QUANT_CASES = [
    # B, H, N, D, scale_block, hadamard, seed, kind
    (1, 2, 256, 64, 64, True, 0x5EED, "iid"),
    (2, 3, 300, 128, 128, True, 7, "outlier"),
    (1, 2, 200, 128, 64, False, 1, "iid"),
    (1, 1, 65, 64, 128, True, 2 ** 64 - 1, "iid"),
    (2, 2, 1, 128, 128, True, 3, "iid"),
    (1, 4, 513, 128, 128, True, 0x5EED, "channel"),
    (1, 2, 130, 64, 64, False, 9, "outlier"),
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "B{}H{}N{}D{}sb{}had{}".format(*c[:6]))
def test_quantize_bit_exact(case):
    B, H, N, D, sb, had, seed, kind = case
    q, k, v = workloads.generate(kind, B, H, N, D, 100 + N)
    got = [host(t) for t in gpu_quantize(q, k, v, sb, had, seed)]
    ref = oq.quantize_qkv(q, k, v, sb, had, seed)
    names = ("q8", "k8", "v8", "q_descale", "k_descale", "v_descale")
    for g, r, nm in zip(got, ref, names):
        assert g.shape == r.shape, nm
        if g.dtype == np.uint8:
            bad = np.count_nonzero(g != r)
            assert bad == 0, f"{nm}: {bad} codes differ"
        else:
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{nm}: descales differ"


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "B{}H{}N{}D{}sb{}had{}".format(*c[:6]))
def test_quantize_pow2_scales_bit_exact(case):
    B, H, N, D, sb, had, seed, kind = case
    q, k, v = workloads.generate(kind, B, H, N, D, 500 + N)
    out = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=sb, hadamard=had, seed=seed, mx=True)
    torch.cuda.synchronize()
    ref = oq.quantize_qkv(q, k, v, sb, had, seed, pow2=True)
    for g, r, nm in zip((host(t) for t in out), ref, ("q8", "k8", "v8", "qd", "kd", "vd")):
        if r.dtype == np.uint8:
            assert np.array_equal(g, r), f"{case} {nm}: {np.count_nonzero(g != r)} codes differ"
        else:
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{case} {nm}"


@pytest.mark.parametrize("pow2", [False, True])
def test_quantize_zero_and_extreme_blocks(pow2):
    B, H, N, D, sb = 1, 2, 256, 128, 128
    q, k, v = workloads.generate("iid", B, H, N, D, 5)
    v[0, 0, :128] = 0.0                      # an all-zero block: descale 1, zero codes
    v[0, 0, 128:200] = -0.0
    q[0, 1, 5, 7] = 3.0e4                    # a huge outlier
    k[0, 1, 130:, :] *= 1e-30                # tiny values: subnormal e4m3 codes
    if pow2:
        # the scale exponent clamps at -127 (the amax / 448 rule would overflow
        # inv = 448 / amax below amax ~ 1.3e-36, outside its contract)
        v[0, 1, 128:, :] *= 1e-38
    out = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=sb, hadamard=True, seed=11, mx=pow2)
    torch.cuda.synchronize()
    got = [host(t) for t in out]
    ref = oq.quantize_qkv(q, k, v, sb, True, 11, pow2=pow2)
    for g, r in zip(got, ref):
        assert np.array_equal(g.view(np.uint8) if g.dtype == np.uint8 else g.view(np.uint32),
                              r.view(np.uint8) if r.dtype == np.uint8 else r.view(np.uint32))


ATTN_CASES = [
    # B, H, N, D, scale_block, hadamard, causal, kind
    (1, 2, 256, 64, 64, True, False, "iid"),
    (1, 2, 256, 64, 64, True, True, "iid"),
    (2, 2, 300, 128, 128, True, False, "outlier"),
    (2, 2, 300, 128, 128, True, True, "outlier"),
    (1, 2, 1000, 128, 64, True, True, "iid"),
    (1, 1, 1, 128, 128, True, False, "iid"),
    (1, 1, 1, 64, 64, False, True, "iid"),
    (1, 2, 129, 64, 128, False, False, "iid"),
    (1, 3, 700, 128, 128, False, True, "channel"),
    (1, 2, 640, 128, 128, True, True, "channel"),
    # scores that rise along the keys: the reference moves on tile after tile,
    # so the loop takes the tile maximum before the exponentials
    (1, 2, 700, 128, 128, True, True, "ramp"),
    (1, 2, 640, 64, 64, False, False, "ramp"),
]


def _fp8_run(q, k, v, sb, had, causal, seed=0x5EED):
    q8, k8, v8, qd, kd, vd = gpu_quantize(q, k, v, sb, had, seed)
    o, lse = fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=sb, hadamard=had, causal=causal)
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "B{}H{}N{}D{}sb{}had{}c{}-{}".format(*c[:8]))
def test_attn_fp8_matches_e1(case):
    B, H, N, D, sb, had, causal, kind = case
    q, k, v = workloads.generate(kind, B, H, N, D, 200 + N)
    o, lse = _fp8_run(q, k, v, sb, had, causal)
    qq = oq.quantize_qkv(q, k, v, sb, had, 0x5EED)
    check_fp8_vs_e1(o, lse, oatt.emulated_fp8_attention_bars(*qq, sb, had, causal), tag=str(case))
    o2, _ = oatt.emulated_fp8_attention_tiled(*qq, sb, had, causal)
    print(f"{case}: diagnostic RMSE vs E2 {rms(o - o2):.3e}")


# Schraudolph's bit-level exponential (attn_fp8_fwd_opts, ATTN_FP8_EXP2_SCHRAUDOLPH)
# against E1, with the bars widened by what the approximation can move O and LSE.
@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "B{}H{}N{}D{}sb{}had{}c{}-{}".format(*c[:8]))
def test_attn_fp8_schraudolph_matches_e1(case):
    B, H, N, D, sb, had, causal, kind = case
    q, k, v = workloads.generate(kind, B, H, N, D, 200 + N)
    q8, k8, v8, qd, kd, vd = gpu_quantize(q, k, v, sb, had, 0x5EED)
    o, lse = fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=sb, hadamard=had, causal=causal,
                             exp2="schraudolph")
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    qq = oq.quantize_qkv(q, k, v, sb, had, 0x5EED)
    check_fp8_vs_e1(o, lse, oatt.emulated_fp8_attention_bars(*qq, sb, had, causal, exp2="schraudolph"),
                    tag=f"{case} schraudolph")
    o2, _ = oatt.emulated_fp8_attention_tiled(*qq, sb, had, causal, exp2="schraudolph")
    print(f"{case}: diagnostic RMSE vs its E2 {rms(o - o2):.3e}")


# Power-of-two block scales applied by the scaled FP8 MFMA (ATTN_FP8_MX), alone
# and with the Schraudolph exponential, against E1 of the power-of-two codes.
MX_CASES = [c + ("exact",) for c in ATTN_CASES] + [c + ("schraudolph",) for c in ATTN_CASES[2:5]]


@pytest.mark.parametrize("case", MX_CASES, ids=lambda c: "B{}H{}N{}D{}sb{}had{}c{}-{}".format(*c[:7], c[8]))
def test_attn_fp8_mx_matches_e1(case):
    B, H, N, D, sb, had, causal, kind, exp2 = case
    q, k, v = workloads.generate(kind, B, H, N, D, 300 + N)
    q8, k8, v8, qd, kd, vd = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=sb, hadamard=had,
                                                 seed=0x5EED, mx=True)
    o, lse = fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=sb, hadamard=had, causal=causal,
                             exp2=exp2, mx=True)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    qq = oq.quantize_qkv(q, k, v, sb, had, 0x5EED, pow2=True)
    check_fp8_vs_e1(o, lse, oatt.emulated_fp8_attention_bars(*qq, sb, had, causal, exp2=exp2), tag=f"{case} mx")
    orf, _ = oatt.reference_attention(q, k, v, causal)
    print(f"{case}: mx RMSE vs FP64 {rms(o - orf):.3e}")


# One power-of-two scale per block x 32 channels (ATTN_FP8_MX32), the MX
# block size: quantiser bit-exact, attention against E1 of those codes.
@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "B{}H{}N{}D{}sb{}had{}".format(*c[:6]))
def test_quantize_mx32_bit_exact(case):
    B, H, N, D, sb, had, seed, kind = case
    q, k, v = workloads.generate(kind, B, H, N, D, 700 + N)
    out = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=sb, hadamard=had, seed=seed, mx32=True)
    torch.cuda.synchronize()
    ref = oq.quantize_qkv(q, k, v, sb, had, seed, pow2=True, group=32)
    for g, r, nm in zip((host(t) for t in out), ref, ("q8", "k8", "v8", "qd", "kd", "vd")):
        assert g.shape == r.shape, nm
        if r.dtype == np.uint8:
            assert np.array_equal(g, r), f"{case} {nm}: {np.count_nonzero(g != r)} codes differ"
        else:
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{case} {nm}"


MX32_CASES = [c + ("exact",) for c in ATTN_CASES] + [c + ("schraudolph",) for c in ATTN_CASES[2:5]]


@pytest.mark.parametrize("case", MX32_CASES, ids=lambda c: "B{}H{}N{}D{}sb{}had{}c{}-{}".format(*c[:7], c[8]))
def test_attn_fp8_mx32_matches_e1(case):
    B, H, N, D, sb, had, causal, kind, exp2 = case
    q, k, v = workloads.generate(kind, B, H, N, D, 800 + N)
    qq_gpu = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=sb, hadamard=had, seed=0x5EED, mx32=True)
    o, lse = fa.attn_fp8_fwd(*qq_gpu, scale_block=sb, hadamard=had, causal=causal, exp2=exp2, mx32=True)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    qq = oq.quantize_qkv(q, k, v, sb, had, 0x5EED, pow2=True, group=32)
    check_fp8_vs_e1(o, lse, oatt.emulated_fp8_attention_bars(*qq, sb, had, causal, exp2=exp2), tag=f"{case} mx32")
    orf, _ = oatt.reference_attention(q, k, v, causal)
    print(f"{case}: mx32 RMSE vs FP64 {rms(o - orf):.3e}")


BF16_CASES = [
    (1, 2, 256, 64, False), (1, 2, 256, 64, True), (2, 2, 300, 128, False), (2, 2, 300, 128, True),
    (1, 1, 1, 128, True), (1, 2, 1000, 128, True), (1, 1, 65, 64, False),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "B{}H{}N{}D{}c{}".format(*c))
def test_attn_bf16_matches_reference(case):
    B, H, N, D, causal = case
    q, k, v = workloads.generate("iid", B, H, N, D, 300 + N)
    qb, kb, vb = (bf16_round(x) for x in (q, k, v))
    to16 = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    o, lse = fa.attn_bf16_fwd(to16(qb), to16(kb), to16(vb), causal=causal)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    o_ref, lse_ref = oatt.reference_attention(qb, kb, vb, causal)
    err = np.abs(o - o_ref)
    # P rounded to BF16 (relative 2^-9) inside the weighted sum moves O by at most
    # 2^-9 max|V|; the result is rounded to BF16 (relative 2^-9); FP32 accumulation
    # and the hardware exp2/log2 add far less.
    vmax = np.abs(vb).max(axis=(-2, -1), keepdims=True)
    assert np.all(err <= 2.0 ** -9 * vmax + 2.0 ** -8 * np.abs(o_ref) + 1e-6), float(err.max())
    assert rms(o - o_ref) <= 2.0 ** -9 * (rms(o_ref) + rms(vb))
    assert np.all(np.abs(lse - lse_ref) <= 1e-4 * np.maximum(1.0, np.abs(lse_ref)))


def test_fp8_run_to_run_bitwise_deterministic():
    q, k, v = workloads.generate("outlier", 1, 4, 1000, 128, 17)
    o1, l1 = _fp8_run(q, k, v, 128, True, True)
    o2, l2 = _fp8_run(q, k, v, 128, True, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


def test_fp8_causal_output_ignores_later_scale_blocks():
    # block scales make O_i depend on later tokens of its own block only (never on later blocks)
    q, k, v = workloads.generate("iid", 1, 2, 512, 128, 23)
    o1, l1 = _fp8_run(q, k, v, 128, True, True)
    k2, v2 = k.copy(), v.copy()
    k2[..., 256:, :] *= 7.0
    v2[..., 256:, :] *= -3.0
    o2, l2 = _fp8_run(q, k2, v2, 128, True, True)
    assert np.array_equal(o1[..., :256, :], o2[..., :256, :])
    assert np.array_equal(l1[..., :256], l2[..., :256])


def test_outputs_on_current_stream():
    q, k, v = workloads.generate("iid", 1, 2, 256, 128, 29)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q8, k8, v8, qd, kd, vd = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=128)
        o, lse = fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=128)
    s.synchronize()
    o_ref, _ = _fp8_run(q, k, v, 128, True, False)
    assert np.array_equal(host(o), o_ref)
