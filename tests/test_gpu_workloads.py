"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  The oracle checks what it can compute piece by piece: the
quantiser bit-exactly on every (batch, head) slice (blocks never cross heads),
and O / LSE on sampled query rows of every head (always rows 0, 1, 127, 128,
N/2 and N-1) against E1, the exact attention of the quantised inputs, with
the bars of ``tests.gpu_common.check_fp8_vs_e1``.  The options (Schraudolph's
exponential, power-of-two scales on the scaled matrix cores) are checked on
eight heads of the outlier workloads.
"""

import numpy as np
import pytest
import torch

import fp8_attention_forward_amd as fa
import workloads
from oracle import attention as oatt
from tests.gpu_common import bf16_round, check_heads_vs_e1, dev, host, rms, sample_rows

pytestmark = [pytest.mark.gpu, pytest.mark.slow,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

NAMES = ["tiny", "outlier", "outlier_causal", "ablation", "ablation_tail", "channel", "channel_norot"]


def _all_heads(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


def _some_heads(w, count=8):
    rng = np.random.default_rng(w.B * 100 + w.H)
    hs = {(0, 0), (w.B - 1, w.H - 1)}
    for i in rng.choice(w.B * w.H, size=min(count, w.B * w.H), replace=False):
        hs.add((int(i) // w.H, int(i) % w.H))
    return sorted(hs)[:max(count, 2)]


def _run(w, q, k, v, exp2="exact", mx=False, mx32=False):
    out = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=w.scale_block, hadamard=w.hadamard,
                              seed=w.sign_seed, mx=mx, mx32=mx32)
    o, lse = fa.attn_fp8_fwd(*out, scale_block=w.scale_block, hadamard=w.hadamard, causal=w.causal, exp2=exp2, mx=mx,
                             mx32=mx32)
    torch.cuda.synchronize()
    return [host(t) for t in out] + [host(o), host(lse)]


@pytest.mark.parametrize("name", NAMES)
def test_workload_fp8_parity(name):
    w = workloads.WORKLOADS[name]
    print(f"\n[{name}] generating {w.B}x{w.H}x{w.N}x{w.D}", flush=True)
    q, k, v = workloads.generate_workload(w)
    print(f"[{name}] quantise + attention on the GPU", flush=True)
    got = _run(w, q, k, v)
    res = check_heads_vs_e1(name, (q, k, v), got, _all_heads(w), w.scale_block, w.hadamard, w.causal, w.sign_seed)
    r = np.array(res)
    print(f"[{name}] {len(res)} heads: RMSE vs E1 median {np.median(r[:, 0]):.3e} max {r[:, 0].max():.3e}; "
          f"max err {r[:, 1].max():.3e}", flush=True)
    # the diagnostic: the kernel-shaped loop E2 on one head
    from oracle import quantize as oq
    sl = (slice(0, 1), slice(0, 1))
    ref = oq.quantize_qkv(q[sl], k[sl], v[sl], w.scale_block, w.hadamard, w.sign_seed)
    rows = sample_rows(w.N, 4, seed=0)
    o2, _ = oatt.emulated_fp8_attention_tiled(*ref, w.scale_block, w.hadamard, w.causal, rows=rows)
    orf, _ = oatt.reference_attention(q[sl], k[sl], v[sl], w.causal, rows=rows)
    og = got[6][sl][..., rows, :]
    print(f"[{name}] head (0, 0) diagnostics: vs E2 rmse {rms(og - o2):.3e}; vs FP64 rmse {rms(og - orf):.3e}",
          flush=True)


@pytest.mark.parametrize("exp2,mx", [("schraudolph", False), ("exact", True), ("schraudolph", True)])
@pytest.mark.parametrize("name", ["outlier", "outlier_causal"])
def test_workload_fp8_options_parity(name, exp2, mx):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.generate_workload(w)
    print(f"\n[{name} {exp2} mx={mx}] quantise + attention on the GPU", flush=True)
    got = _run(w, q, k, v, exp2=exp2, mx=mx)
    res = check_heads_vs_e1(f"{name} {exp2} mx={mx}", (q, k, v), got, _some_heads(w), w.scale_block, w.hadamard,
                            w.causal, w.sign_seed, exp2=exp2, mx=mx)
    r = np.array(res)
    print(f"[{name} {exp2} mx={mx}] RMSE vs E1 max {r[:, 0].max():.3e}, max err {r[:, 1].max():.3e}", flush=True)


@pytest.mark.parametrize("name", ["outlier", "channel_norot"])
def test_workload_fp8_mx32_parity(name):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.generate_workload(w)
    print(f"\n[{name} mx32] quantise + attention on the GPU", flush=True)
    got = _run(w, q, k, v, mx32=True)
    res = check_heads_vs_e1(f"{name} mx32", (q, k, v), got, _some_heads(w), w.scale_block, w.hadamard, w.causal,
                            w.sign_seed, group=32)
    r = np.array(res)
    print(f"[{name} mx32] RMSE vs E1 max {r[:, 0].max():.3e}, max err {r[:, 1].max():.3e}", flush=True)


@pytest.mark.parametrize("name", ["outlier", "outlier_causal", "ablation_tail"])
def test_workload_bf16_parity(name):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.generate_workload(w)
    to16 = lambda x: dev(x).to(torch.bfloat16)
    qb, kb, vb = to16(q), to16(k), to16(v)
    o, lse = fa.attn_bf16_fwd(qb, kb, vb, causal=w.causal)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    for (b, h) in _some_heads(w):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rows = sample_rows(w.N, 24, seed=b * 1000 + h)
        qr, kr, vr = (bf16_round(x[sl]) for x in (q, k, v))
        orf, lrf = oatt.reference_attention(qr, kr, vr, w.causal, rows=rows)
        og = o[sl][..., rows, :]
        lg = lse[sl][..., rows]
        vmax = np.abs(vr).max()
        assert np.all(np.abs(og - orf) <= 2.0 ** -9 * vmax + 2.0 ** -8 * np.abs(orf) + 1e-6)
        assert np.all(np.abs(lg - lrf) <= 1e-4 * np.maximum(1.0, np.abs(lrf)))
        print(f"[{name} bf16] head {(b, h)}: rmse {rms(og - orf):.3e} max {np.max(np.abs(og - orf)):.3e}", flush=True)
