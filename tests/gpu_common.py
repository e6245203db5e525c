"""Helpers for the GPU parity tests: run the HIP path through the binding, run
the oracle on the same seeded inputs, and compare."""

import math

import numpy as np
import torch

import fp8_attention_forward_amd as fa

# Tolerances of the FP8 path against the emulation of the same pipeline
# (oracle E2, whose O is rounded to BF16 as the kernel's is).  RMSE and
# max-abs bounds on O; the max-abs bound adds one BF16 ulp of the reference
# value, because a float32 result a hair away from the float64 one can round
# to the neighbouring BF16 value (a bound of 2e-2 alone is below one BF16 ulp
# wherever |O| >= 2.56).
FP8_RMSE_TOL = 2e-3
FP8_MAX_TOL = 2e-2
LSE_REL_TOL = 2e-3


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bf16_round(x):
    """float32 -> bfloat16 -> float32 (round to nearest even), via torch on the CPU."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def ulp_bf16(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def gpu_quantize(q, k, v, sb, hadamard, seed):
    out = fa.quantize_qkv_fp8(dev(q), dev(k), dev(v), scale_block=sb, hadamard=hadamard, seed=seed)
    torch.cuda.synchronize()
    return out


def check_fp8_output(o_gpu, lse_gpu, o_ref, lse_ref, tag="", slack=None):
    """RMSE and max-abs bounds on O, relative bound on LSE.

    ``slack`` (the oracle's tie slack, same shape as O) widens the max-abs
    bound element by element by what valid roundings of P at float32 precision
    can move O: a P whose exact value sits on an e4m3 rounding midpoint may
    round either way in the kernel."""
    err = o_gpu - o_ref
    rmse = float(np.sqrt(np.mean(err ** 2)))
    tol = FP8_MAX_TOL + ulp_bf16(o_ref)
    strict = np.abs(err) > tol
    if slack is not None:
        tol = tol + slack
    worst = float(np.max(np.abs(err) - tol))
    assert rmse <= FP8_RMSE_TOL, f"{tag}: RMSE {rmse:.3e} > {FP8_RMSE_TOL}"
    assert worst <= 0, f"{tag}: max |err| exceeds bound by {worst:.3e} (max err {np.max(np.abs(err)):.3e})"
    if slack is not None and strict.any():
        print(f"{tag}: {int(strict.sum())} element(s) beyond {FP8_MAX_TOL} within the tie slack "
              f"(max err {float(np.max(np.abs(err))):.3e})", flush=True)
    lerr = np.abs(lse_gpu - lse_ref)
    assert np.all(lerr <= LSE_REL_TOL * np.maximum(1.0, np.abs(lse_ref))), f"{tag}: LSE err {lerr.max():.3e}"
    return rmse, float(np.max(np.abs(err)))


def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    base = {0, 1, n - 1, n // 2, min(n - 1, 127), min(n - 1, 128)}
    extra = rng.choice(n, size=min(n, count), replace=False)
    return np.array(sorted(base | set(int(x) for x in extra)), dtype=np.int64)


def rms(x):
    return float(math.sqrt(np.mean(np.asarray(x, dtype=np.float64) ** 2)))
