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


def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    base = {0, 1, n - 1, n // 2, min(n - 1, 127), min(n - 1, 128)} & set(range(n))
    extra = rng.choice(n, size=min(n, count), replace=False)
    return np.array(sorted(base | set(int(x) for x in extra)), dtype=np.int64)


def rms(x):
    return float(math.sqrt(np.mean(np.asarray(x, dtype=np.float64) ** 2)))


def check_fp8_vs_e1(o_gpu, lse_gpu, bars, tag=""):
    """Assert the FP8 contract against E1, with the bars of
    ``oracle.attention.emulated_fp8_attention_bars`` (same shapes as O / LSE):

      max |dO| <= max(2e-2, pbar) + acc_bar + half a BF16 ulp of the output
      RMSE     <= max(2e-3, 2 rms(sigma)) + rms(acc_bar)
      |dLSE|   <= 2e-3 max(1, |LSE|) + lse_bar

    Returns (rmse, max error, RMSE bar)."""
    o1, l1 = bars["o"], bars["lse"]
    err = np.asarray(o_gpu, dtype=np.float64) - o1
    mag = np.maximum(np.abs(o_gpu), np.abs(o1))
    tol = np.maximum(FP8_MAX_TOL, bars["pbar"]) + bars["acc_bar"] + 0.5 * ulp_bf16(mag)
    over = np.abs(err) - tol
    rmse = float(np.sqrt(np.mean(err ** 2)))
    rmse_bar = max(FP8_RMSE_TOL, 2.0 * float(np.sqrt(np.mean(bars["sigma"] ** 2)))) + rms(bars["acc_bar"])
    wide = int(np.count_nonzero(np.abs(err) > FP8_MAX_TOL + 0.5 * ulp_bf16(mag)))
    print(f"{tag}: vs E1 RMSE {rmse:.3e} (bar {rmse_bar:.3e}), max err {float(np.max(np.abs(err))):.3e}, "
          f"{wide} element(s) beyond 2e-2 inside the derived bar", flush=True)
    assert rmse <= rmse_bar, f"{tag}: RMSE vs E1 {rmse:.3e} > {rmse_bar:.3e}"
    assert np.all(over <= 0), (f"{tag}: |O - E1| exceeds its bar by {float(over.max()):.3e} "
                               f"(max err {float(np.max(np.abs(err))):.3e})")
    lerr = np.abs(np.asarray(lse_gpu, dtype=np.float64) - l1)
    lbar = LSE_REL_TOL * np.maximum(1.0, np.abs(l1)) + bars["lse_bar"]
    assert np.all(lerr <= lbar), f"{tag}: LSE err {float(lerr.max()):.3e} beyond its bar"
    return rmse, float(np.max(np.abs(err))), rmse_bar


def check_heads_vs_e1(name, x_host, got_host, heads, scale_block, hadamard, causal, sign_seed, n_rows=4,
                      exp2="exact", mx=False, workers=8, group=None):
    """Full-size parity on whole heads: for every (b, h) in ``heads`` the
    oracle quantises that head (blocks never cross heads), the GPU codes and
    descales must equal it bit for bit, and O / LSE on sampled rows (always
    rows 0, 1, 127, 128, N/2 and N-1) must meet the E1 bars.  The heads run in
    a thread pool (numpy releases the interpreter lock in its heavy parts).

    x_host: (q, k, v) float32 [B, H, N, D]; got_host: (q8, k8, v8, qd, kd, vd,
    o, lse) as numpy arrays.  Returns the per-head (rmse, max err, bar)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import attention as oatt
    from oracle import quantize as oq
    q, k, v = x_host
    n = q.shape[2]

    def one(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oq.quantize_qkv(q[sl], k[sl], v[sl], scale_block, hadamard, sign_seed, pow2=mx or group is not None,
                              group=group)
        for g, r, nm in zip(got_host[:6], ref, ("q8", "k8", "v8", "qd", "kd", "vd")):
            g = g[sl]
            same = np.array_equal(g, r) if r.dtype == np.uint8 else np.array_equal(g.view(np.uint32), r.view(np.uint32))
            assert same, f"{name} head {bh}: {nm} differs from the oracle quantiser"
        rows = sample_rows(n, n_rows, seed=b * 1000 + h)
        bars = oatt.emulated_fp8_attention_bars(*ref, scale_block, hadamard, causal, rows=rows, exp2=exp2)
        og = got_host[6][sl][..., rows, :]
        lg = got_host[7][sl][..., rows]
        return check_fp8_vs_e1(og, lg, bars, tag=f"[{name}] head {bh}")

    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(one, heads))
