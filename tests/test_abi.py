"""The C-ABI library: it loads without a GPU, exports what include/attn_fp8.h
declares, and rejects bad arguments before touching the device."""

import ctypes
import os
import re
import subprocess

import pytest

import fp8_attention_forward_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_fp8.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail(f"{fa.LIB_PATH} missing: run `python -m fp8_attention_forward_amd.build`")
    return fa.load_library()


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(line.split()[-1] for line in out.stdout.splitlines() if line.strip())
    for name in _declared_functions():
        assert name in exported, name


def test_abi_version(lib):
    assert fa.abi_version() == 2
    m = re.search(r"#define ATTN_FP8_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == fa.abi_version()


# Fake, never-dereferenced device addresses: every call below must fail validation
# before any HIP call is made.
P = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10008)        # 8-byte aligned only
NUL = ctypes.c_void_p(0)


def _q(lib, **kw):
    a = dict(q=P, k=P, v=P, B=1, H=1, N=64, D=128, sb=128, had=1, seed=1, q8=P, k8=P, v8=P, qd=P, kd=P, vd=P)
    a.update(kw)
    return lib.quantize_qkv_fp8(a["q"], a["k"], a["v"], a["B"], a["H"], a["N"], a["D"], a["sb"], a["had"],
                                a["seed"], a["q8"], a["k8"], a["v8"], a["qd"], a["kd"], a["vd"], None)


def _a(lib, **kw):
    a = dict(q8=P, k8=P, v8=P, qd=P, kd=P, vd=P, B=1, H=1, N=64, D=128, sb=128, had=1, causal=0, o=P, lse=P)
    a.update(kw)
    return lib.attn_fp8_fwd(a["q8"], a["k8"], a["v8"], a["qd"], a["kd"], a["vd"], a["B"], a["H"], a["N"], a["D"],
                            a["sb"], a["had"], a["causal"], a["o"], a["lse"], None)


def _b(lib, **kw):
    a = dict(q=P, k=P, v=P, B=1, H=1, N=64, D=128, causal=0, o=P, lse=P)
    a.update(kw)
    return lib.attn_bf16_fwd(a["q"], a["k"], a["v"], a["B"], a["H"], a["N"], a["D"], a["causal"], a["o"],
                             a["lse"], None)


@pytest.mark.parametrize("kw,frag", [
    (dict(D=96), "D must be 64 or 128"),
    (dict(D=256), "D must be 64 or 128"),
    (dict(N=0), ">= 1"),
    (dict(B=-1), ">= 1"),
    (dict(sb=32), "scale_block"),
    (dict(q=NUL), "q is NULL"),
    (dict(v8=MIS), "v8 is not 16-byte aligned"),
    (dict(kd=NUL), "k_descale is NULL"),
    (dict(B=1 << 20, H=1 << 12), "2^31"),
])
def test_quantize_rejects(lib, kw, frag):
    assert _q(lib, **kw) == fa.ATTN_EINVAL
    assert frag in fa.last_error()


@pytest.mark.parametrize("kw,frag", [
    (dict(D=32), "D must be 64 or 128"),
    (dict(sb=0), "scale_block"),
    (dict(o=MIS), "o_bf16 is not 16-byte aligned"),
    (dict(lse=NUL), "lse is NULL"),
    (dict(k8=NUL), "k8 is NULL"),
    (dict(H=0), ">= 1"),
])
def test_attn_fp8_rejects(lib, kw, frag):
    assert _a(lib, **kw) == fa.ATTN_EINVAL
    assert frag in fa.last_error()


def test_attn_fp8_opts_rejects_unknown_flags(lib):
    args = [P, P, P, P, P, P, 1, 1, 64, 128, 128, 1, 0]
    assert lib.attn_fp8_fwd_opts(*args, 4, P, P, None) == fa.ATTN_EINVAL
    assert "unknown flags" in fa.last_error()
    assert lib.attn_fp8_fwd_opts(*args, 3, NUL, P, None) == fa.ATTN_EINVAL   # both options known: next check
    assert "o_bf16 is NULL" in fa.last_error()
    assert lib.attn_fp8_fwd_opts(*args, 1, NUL, P, None) == fa.ATTN_EINVAL   # valid flag, then validation
    assert "o_bf16 is NULL" in fa.last_error()
    m = re.search(r"#define ATTN_FP8_EXP2_SCHRAUDOLPH (\d+)u", open(HEADER).read())
    assert int(m.group(1)) == fa.ATTN_FP8_EXP2_SCHRAUDOLPH


def test_quantize_opts_flags(lib):
    a = [P, P, P, 1, 1, 64, 128, 128, 1, 1]
    assert lib.quantize_qkv_fp8_opts(*a, 1, P, P, P, P, P, P, None) == fa.ATTN_EINVAL   # EXP2 is not a quantiser flag
    assert "unknown flags" in fa.last_error()
    assert lib.quantize_qkv_fp8_opts(*a, 2, P, P, NUL, P, P, P, None) == fa.ATTN_EINVAL
    assert "v8 is NULL" in fa.last_error()
    m = re.search(r"#define ATTN_FP8_MX (\d+)u", open(HEADER).read())
    assert int(m.group(1)) == fa.ATTN_FP8_MX


def test_rejects_heads_too_long_for_32_bit_offsets(lib):
    assert _a(lib, N=1 << 23, D=128) == fa.ATTN_EINVAL
    assert "N * D" in fa.last_error()


@pytest.mark.parametrize("kw,frag", [
    (dict(D=80), "D must be 64 or 128"),
    (dict(q=MIS), "q is not 16-byte aligned"),
    (dict(o=NUL), "o_bf16 is NULL"),
])
def test_attn_bf16_rejects(lib, kw, frag):
    assert _b(lib, **kw) == fa.ATTN_EINVAL
    assert frag in fa.last_error()


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError, match="device tensor"):
        fa.quantize_qkv_fp8(x, x, x, scale_block=64)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        fa.load_library(str(tmp_path / "missing.so"))
