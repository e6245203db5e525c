"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  The oracle checks sampled outputs it can compute one by one:
the quantiser bit-exactly on sampled (batch, head) slices (blocks are
independent per head), and O / LSE on sampled query rows of those heads.
"""

import numpy as np
import pytest
import torch

import fp8_attention_forward_amd as fa
import workloads
from oracle import attention as oatt
from oracle import quantize as oq
from tests.gpu_common import (FP8_MAX_TOL, FP8_RMSE_TOL, bf16_round, check_fp8_output, dev, host,
                              rms, sample_rows)

pytestmark = [pytest.mark.gpu, pytest.mark.slow,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

NAMES = ["tiny", "outlier", "outlier_causal", "ablation", "ablation_tail", "channel", "channel_norot"]

# Without the rotation, the channel-outlier inputs put one huge product into a
# group of eight channels; the FP8 matrix cores of gfx950 sum each group of
# eight products aligned to its largest term with about 13 fractional bits
# (measured), so the other seven channels of that group lose their low bits in
# S.  That error is a property of FP8 accumulation on this hardware, not of
# the loop; it is bounded here by a looser tolerance, and the rotation (the
# method) removes it.
LOOSE = {"channel_norot": dict(rmse=2e-2, lse=2e-2)}


def _heads(w):
    hs = {(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 2)}
    return sorted(hs)


@pytest.fixture(scope="module")
def cache():
    return {}


@pytest.mark.parametrize("name", NAMES)
def test_workload_fp8_parity(name, cache):
    w = workloads.WORKLOADS[name]
    print(f"\n[{name}] generating {w.B}x{w.H}x{w.N}x{w.D}", flush=True)
    q, k, v = workloads.generate_workload(w)
    print(f"[{name}] quantise + attention on the GPU", flush=True)
    q8, k8, v8, qd, kd, vd = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=w.scale_block,
                                                 hadamard=w.hadamard, seed=w.sign_seed)
    o, lse = fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=w.scale_block, hadamard=w.hadamard,
                             causal=w.causal)
    torch.cuda.synchronize()
    loose = LOOSE.get(name)
    for (b, h) in _heads(w):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oq.quantize_qkv(q[sl], k[sl], v[sl], w.scale_block, w.hadamard, w.sign_seed)
        got = [host(t[sl]) for t in (q8, k8, v8, qd, kd, vd)]
        for g, r, nm in zip(got, ref, ("q8", "k8", "v8", "qd", "kd", "vd")):
            if g.dtype == np.uint8:
                assert np.array_equal(g, r), f"{name} head {(b, h)}: {nm} differs in {np.count_nonzero(g != r)} codes"
            else:
                assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{name} head {(b, h)}: {nm}"
        rows = sample_rows(w.N, 24, seed=b * 1000 + h)
        o2, l2, slk = oatt.emulated_fp8_attention_tiled(*ref, w.scale_block, w.hadamard, w.causal, rows=rows,
                                                        tie_slack=True)
        og = host(o[sl])[..., rows, :]
        lg = host(lse[sl])[..., rows]
        if loose is None:
            r2, m2 = check_fp8_output(og, lg, o2, l2, tag=f"{name} head {(b, h)}", slack=slk)
        else:
            r2 = rms(og - o2)
            m2 = float(np.max(np.abs(og - o2)))
            assert r2 <= loose["rmse"], f"{name}: RMSE {r2:.3e}"
            assert np.all(np.abs(lg - l2) <= loose["lse"] * np.maximum(1.0, np.abs(l2)))
        o1, _ = oatt.emulated_fp8_attention(*ref, w.scale_block, w.hadamard, w.causal, rows=rows)
        orf, _ = oatt.reference_attention(q[sl], k[sl], v[sl], w.causal, rows=rows)
        print(f"[{name}] head {(b, h)}: vs E2 rmse {r2:.3e} max {m2:.3e}; vs E1 rmse {rms(og - o1):.3e}; "
              f"vs FP64 rmse {rms(og - orf):.3e}; RMS(O) {rms(orf):.3e}", flush=True)


@pytest.mark.parametrize("name", ["outlier", "outlier_causal"])
def test_workload_fp8_schraudolph_parity(name):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.generate_workload(w)
    q8, k8, v8, qd, kd, vd = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=w.scale_block,
                                                 hadamard=w.hadamard, seed=w.sign_seed)
    o, lse = fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=w.scale_block, hadamard=w.hadamard,
                             causal=w.causal, exp2="schraudolph")
    torch.cuda.synchronize()
    for (b, h) in _heads(w):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oq.quantize_qkv(q[sl], k[sl], v[sl], w.scale_block, w.hadamard, w.sign_seed)
        rows = sample_rows(w.N, 24, seed=b * 1000 + h)
        o2, l2, slk = oatt.emulated_fp8_attention_tiled(*ref, w.scale_block, w.hadamard, w.causal, rows=rows,
                                                        exp2="schraudolph", tie_slack=True)
        og = host(o[sl])[..., rows, :]
        lg = host(lse[sl])[..., rows]
        r2, m2 = check_fp8_output(og, lg, o2, l2, tag=f"{name} schraudolph head {(b, h)}", slack=slk)
        orf, _ = oatt.reference_attention(q[sl], k[sl], v[sl], w.causal, rows=rows)
        print(f"[{name} schraudolph] head {(b, h)}: vs E2 rmse {r2:.3e} max {m2:.3e}; vs FP64 rmse "
              f"{rms(og - orf):.3e}", flush=True)


@pytest.mark.parametrize("name", ["outlier", "outlier_causal"])
def test_workload_fp8_mx_parity(name):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.generate_workload(w)
    q8, k8, v8, qd, kd, vd = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=w.scale_block,
                                                 hadamard=w.hadamard, seed=w.sign_seed, mx=True)
    o, lse = fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=w.scale_block, hadamard=w.hadamard,
                             causal=w.causal, mx=True)
    torch.cuda.synchronize()
    for (b, h) in _heads(w):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oq.quantize_qkv(q[sl], k[sl], v[sl], w.scale_block, w.hadamard, w.sign_seed, pow2=True)
        got = [host(t[sl]) for t in (q8, k8, v8, qd, kd, vd)]
        for g, r, nm in zip(got, ref, ("q8", "k8", "v8", "qd", "kd", "vd")):
            same = np.array_equal(g, r) if g.dtype == np.uint8 else np.array_equal(g.view(np.uint32), r.view(np.uint32))
            assert same, f"{name} mx head {(b, h)}: {nm}"
        rows = sample_rows(w.N, 24, seed=b * 1000 + h)
        o2, l2, slk = oatt.emulated_fp8_attention_tiled(*ref, w.scale_block, w.hadamard, w.causal, rows=rows, mx=True,
                                                        tie_slack=True)
        og = host(o[sl])[..., rows, :]
        lg = host(lse[sl])[..., rows]
        r2, m2 = check_fp8_output(og, lg, o2, l2, tag=f"{name} mx head {(b, h)}", slack=slk)
        orf, _ = oatt.reference_attention(q[sl], k[sl], v[sl], w.causal, rows=rows)
        print(f"[{name} mx] head {(b, h)}: vs E2 rmse {r2:.3e} max {m2:.3e}; vs FP64 rmse {rms(og - orf):.3e}",
              flush=True)


@pytest.mark.parametrize("name", ["outlier", "outlier_causal", "ablation_tail"])
def test_workload_bf16_parity(name):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.generate_workload(w)
    to16 = lambda x: dev(x).to(torch.bfloat16)
    qb, kb, vb = to16(q), to16(k), to16(v)
    o, lse = fa.attn_bf16_fwd(qb, kb, vb, causal=w.causal)
    torch.cuda.synchronize()
    for (b, h) in _heads(w):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rows = sample_rows(w.N, 24, seed=b * 1000 + h)
        qr, kr, vr = (bf16_round(x[sl]) for x in (q, k, v))
        orf, lrf = oatt.reference_attention(qr, kr, vr, w.causal, rows=rows)
        og = host(o[sl])[..., rows, :]
        lg = host(lse[sl])[..., rows]
        vmax = np.abs(vr).max()
        assert np.all(np.abs(og - orf) <= 2.0 ** -9 * vmax + 2.0 ** -8 * np.abs(orf) + 1e-6)
        assert np.all(np.abs(lg - lrf) <= 1e-4 * np.maximum(1.0, np.abs(lrf)))
        print(f"[{name} bf16] head {(b, h)}: rmse {rms(og - orf):.3e} max {np.max(np.abs(og - orf)):.3e}", flush=True)
