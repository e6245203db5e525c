"""attn_fp8_decode_noalloc (no workspace, no allocation; its partials live in
the library's per-GPU scratch array) against attn_fp8_decode with a caller
workspace, through the C ABI: bitwise equal on two calls in a row, the second
smaller than the first (the array keeps the first call's partials), and
sizes beyond the array's limit rejected before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import fp8_attention_forward_amd as fa
import workloads
from tests.gpu_common import dev, host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

CASES = [
    # B, Hq, Hkv, Sq, Ncap, D, scale_block, causal, seqlens, split, kind  (the second is smaller)
    (3, 8, 2, 2, 3000, 128, 128, True, [3000, 1234, 77], 0, "outlier"),
    (1, 4, 4, 1, 500, 64, 64, False, [321], 128, "iid"),
]


def _inputs(case, seed):
    B, Hq, Hkv, Sq, Ncap, D, sb, causal, seqlens, split, kind = case
    q, k, v = workloads.generate_decode(kind, B, Hq, Hkv, Sq, Ncap, D, seed)
    _, k8, v8, _, kd, vd = fa.quantize_qkv_fp8(dev(k), dev(k), dev(v), scale_block=sb, seed=0x5EED)
    q8, _, _, qd, _, _ = fa.quantize_qkv_fp8(dev(q), dev(q), dev(q), scale_block=sb, seed=0x5EED)
    return q8, qd, k8, v8, kd, vd, dev(np.asarray(seqlens, np.int32))


def test_noalloc_decode_equals_the_workspace_call_twice():
    for n, case in enumerate(CASES):
        B, Hq, Hkv, Sq, Ncap, D, sb, causal, seqlens, split, kind = case
        print(f"\n[decode noalloc] call {n}: {case[:9]} split {split}", flush=True)
        args = _inputs(case, 90 + n)
        need = fa.attn_fp8_decode_workspace_bytes(B, Hq, Hkv, Sq, Ncap, D, split)
        assert 0 < need <= fa.DECODE_NOALLOC_MAX_BYTES
        o_ref, l_ref = fa.attn_fp8_decode(*args, scale_block=sb, causal=causal, split=split)
        o = torch.full((B, Hq, Sq, D), 3.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, Hq, Sq), 3.0, dtype=torch.float32, device="cuda")
        fa.attn_fp8_decode_noalloc(*args, out=(o, lse), scale_block=sb, causal=causal, split=split)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {n}: O differs from attn_fp8_decode"
        assert np.array_equal(host(lse).view(np.uint32), host(l_ref).view(np.uint32)), f"call {n}: LSE differs"


def test_noalloc_decode_rejects_sizes_beyond_its_scratch():
    lib = fa.load_library()
    t8 = torch.zeros(64, dtype=torch.uint8, device="cuda")
    tf = torch.zeros(64, dtype=torch.float32, device="cuda")
    ti = torch.ones(64, dtype=torch.int32, device="cuda")
    B, Hq, Hkv, Sq, Ncap, D, split = 8, 256, 8, 1, 65536, 128, 64
    need = fa.attn_fp8_decode_workspace_bytes(B, Hq, Hkv, Sq, Ncap, D, split)
    assert need > fa.DECODE_NOALLOC_MAX_BYTES
    p8, pf, pi = (ctypes.c_void_p(t.data_ptr()) for t in (t8, tf, ti))
    st = lib.attn_fp8_decode_noalloc(p8, pf, p8, p8, pf, pf, pi, B, Hq, Hkv, Sq, Ncap, D, 128, 1, 1, split, p8, pf,
                                     None)
    assert st == fa.ATTN_EINVAL
    assert "scratch" in fa.last_error()
