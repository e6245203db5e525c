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
    assert fa.abi_version() == 5
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


def test_mx32_flag_is_known_to_the_dense_calls_only(lib):
    assert fa.ATTN_FP8_MX32 == int(re.search(r"#define ATTN_FP8_MX32 (\d+)u", open(HEADER).read()).group(1))
    a = [P, P, P, 1, 1, 64, 128, 128, 1, 1]
    # dense: a known flag, so validation goes on to the pointers
    assert lib.quantize_qkv_fp8_opts(*a, fa.ATTN_FP8_MX32, P, P, NUL, P, P, P, None) == fa.ATTN_EINVAL
    assert "v8 is NULL" in fa.last_error()
    args = [P, P, P, P, P, P, 1, 1, 64, 128, 128, 1, 0]
    assert lib.attn_fp8_fwd_opts(*args, fa.ATTN_FP8_MX32, NUL, P, None) == fa.ATTN_EINVAL
    assert "o_bf16 is NULL" in fa.last_error()
    # packed documents: not an option there
    cu = P
    assert lib.quantize_qkv_fp8_varlen(P, P, P, cu, 1, 1, 128, 128, 128, 1, 1, fa.ATTN_FP8_MX32,
                                       P, P, P, P, P, P, None) == fa.ATTN_EINVAL
    assert "unknown flags" in fa.last_error()


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


def _qv(lib, **kw):
    a = dict(q=P, k=P, v=P, cu=P, ndoc=3, H=2, T=1000, D=128, sb=128, had=1, seed=1, flags=0, q8=P, k8=P, v8=P,
             qd=P, kd=P, vd=P)
    a.update(kw)
    return lib.quantize_qkv_fp8_varlen(a["q"], a["k"], a["v"], a["cu"], a["ndoc"], a["H"], a["T"], a["D"], a["sb"],
                                       a["had"], a["seed"], a["flags"], a["q8"], a["k8"], a["v8"], a["qd"], a["kd"],
                                       a["vd"], None)


def _av(lib, **kw):
    a = dict(q8=P, k8=P, v8=P, qd=P, kd=P, vd=P, cu=P, ndoc=3, H=2, T=1000, D=128, sb=128, had=1, causal=1, flags=0,
             ws=P, wsb=1 << 20, o=P, lse=P)
    a.update(kw)
    return lib.attn_fp8_fwd_varlen(a["q8"], a["k8"], a["v8"], a["qd"], a["kd"], a["vd"], a["cu"], a["ndoc"], a["H"],
                                   a["T"], a["D"], a["sb"], a["had"], a["causal"], a["flags"], a["ws"], a["wsb"],
                                   a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,frag", [
    (dict(ndoc=0), ">= 1"),
    (dict(T=0), ">= 1"),
    (dict(T=(1 << 20) + 1), "T must be <= 1048576"),
    (dict(D=96), "D must be 64 or 128"),
    (dict(sb=256), "scale_block"),
    (dict(cu=NUL), "cu_seqlens is NULL"),
    (dict(cu=ctypes.c_void_p(0x10002)), "cu_seqlens is not 4-byte aligned"),
    (dict(flags=1), "unknown flags"),
    (dict(flags=4), "unknown flags"),
    (dict(vd=NUL), "v_descale is NULL"),
    (dict(H=1 << 17, T=1 << 20, sb=64), "2^31"),
])
def test_quantize_varlen_rejects(lib, kw, frag):
    assert _qv(lib, **kw) == fa.ATTN_EINVAL
    assert frag in fa.last_error()


@pytest.mark.parametrize("kw,frag", [
    (dict(ndoc=-1), ">= 1"),
    (dict(ndoc=(1 << 24) + 1), "ndoc must be <= 2^24"),
    (dict(D=32), "D must be 64 or 128"),
    (dict(flags=8), "unknown flags"),
    (dict(ws=NUL), "workspace is NULL"),
    (dict(ws=MIS), "workspace is not 16-byte aligned"),
    (dict(wsb=16 + 8 * ((1000 + 127 * 3) // 128) - 1), "workspace_bytes"),
    (dict(o=MIS), "o_bf16 is not 16-byte aligned"),
    (dict(cu=NUL), "cu_seqlens is NULL"),
    (dict(H=1 << 20, T=1 << 20, ndoc=1000), "2^31"),
])
def test_attn_fp8_varlen_rejects(lib, kw, frag):
    assert _av(lib, **kw) == fa.ATTN_EINVAL
    assert frag in fa.last_error()


def test_varlen_flags_and_workspace_size(lib):
    # every known flag passes the flag check (the NULL output fails next)
    assert _av(lib, flags=7, o=NUL) == fa.ATTN_EINVAL and "o_bf16 is NULL" in fa.last_error()
    assert _qv(lib, flags=2, q8=NUL) == fa.ATTN_EINVAL and "q8 is NULL" in fa.last_error()
    m = re.search(r"#define ATTN_FP8_NATURAL_ORDER (\d+)u", open(HEADER).read())
    assert int(m.group(1)) == fa.ATTN_FP8_NATURAL_ORDER
    # 16 header bytes + 8 per possible item; the items of T tokens in ndoc
    # documents are at most sum ceil(l / 128) <= (T + 127 ndoc) / 128
    assert fa.attn_fp8_varlen_workspace_bytes(1000, 3) == 16 + 8 * ((1000 + 381) // 128)
    assert fa.attn_fp8_varlen_workspace_bytes(128, 1) == 16 + 8
    assert fa.attn_fp8_varlen_workspace_bytes(0, 1) == 0 and fa.attn_fp8_varlen_workspace_bytes(5, 0) == 0
    import itertools
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(200):
        T, nd = int(rng.integers(1, 5000)), int(rng.integers(1, 50))
        cuts = np.sort(rng.integers(0, T + 1, nd - 1))
        lens = np.diff(np.concatenate([[0], cuts, [T]]))
        assert 16 + 8 * int(sum(-(-l // 128) for l in lens)) <= fa.attn_fp8_varlen_workspace_bytes(T, nd)


def _dec(lib, **kw):
    a = dict(q8=P, qd=P, k8=P, v8=P, kd=P, vd=P, sl=P, B=2, Hq=8, Hkv=2, Sq=1, Ncap=4096, D=128, sb=128, had=1,
             causal=1, split=0, ws=P, wsb=1 << 30, o=P, lse=P)
    a.update(kw)
    return lib.attn_fp8_decode(a["q8"], a["qd"], a["k8"], a["v8"], a["kd"], a["vd"], a["sl"], a["B"], a["Hq"],
                               a["Hkv"], a["Sq"], a["Ncap"], a["D"], a["sb"], a["had"], a["causal"], a["split"],
                               a["ws"], a["wsb"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,frag", [
    (dict(B=0), ">= 1"),
    (dict(Ncap=0), ">= 1"),
    (dict(D=80), "D must be 64 or 128"),
    (dict(sb=96), "scale_block"),
    (dict(Hq=6, Hkv=4), "multiple of Hkv"),
    (dict(Hq=64, Hkv=1), "<= 32"),
    (dict(Hq=8, Hkv=2, Sq=9), "<= 32"),
    (dict(Ncap=1 << 23), "Ncap * D"),
    (dict(B=300, Hkv=300, Hq=300), "65535"),
    (dict(split=100), "split"),
    (dict(split=16384), "split"),
    (dict(Ncap=(1 << 24) - 1, D=64, split=64), "65535"),          # split index is the grid's y dimension
    (dict(sl=NUL), "seqlens is NULL"),
    (dict(ws=MIS), "workspace is not 16-byte aligned"),
    (dict(wsb=16), "workspace_bytes"),
    (dict(o=NUL), "o_bf16 is NULL"),
])
def test_attn_fp8_decode_rejects(lib, kw, frag):
    assert _dec(lib, **kw) == fa.ATTN_EINVAL
    assert frag in fa.last_error()


def test_decode_split_and_workspace_size(lib):
    # explicit splits pass through (fixed ranges)
    assert fa.attn_fp8_decode_split(2, 2, 4096, 192) == 192
    # split 0 up to 512 sequences: the balanced shares (no fixed range)
    for B, Hkv, N in ((1, 1, 100), (2, 8, 4096), (16, 8, 32768), (512, 1, 64)):
        assert fa.attn_fp8_decode_split(B, Hkv, N) == 0
    # split 0 above 512 sequences: fixed ranges, a power of two in [64, 1024]
    for B, Hkv, N in ((513, 1, 100), (600, 8, 4096), (1024, 8, 32768), (4096, 1, 1 << 16)):
        s = fa.attn_fp8_decode_split(B, Hkv, N)
        assert s in (64, 128, 256, 512, 1024)
        nsplit = -(-N // (4 * s))
        assert B * Hkv * nsplit >= 1024 or s == 64
        assert s == 1024 or B * Hkv * -(-N // (8 * s)) < 1024          # the largest such power of two
    # partials, (D + 2) floats per query row: balanced shares, one per wave and
    # one per (sequence, K/V head); W = min(2048, tiles of a full cache), a multiple of 4
    for B, Hq, Hkv, Sq, N, D in ((2, 8, 2, 1, 4096, 128), (16, 32, 8, 1, 32768, 128), (1, 1, 1, 1, 64, 64),
                                 (3, 6, 3, 2, 200, 64)):
        W = min(2048, B * Hkv * -(-N // 64))
        W = -(-W // 4) * 4
        assert fa.attn_fp8_decode_workspace_bytes(B, Hq, Hkv, Sq, N, D) == 4 * (W + B * Hkv) * (Hq // Hkv) * Sq * (D + 2)
    # fixed ranges: per (batch, K/V head, range of four waves)
    assert fa.attn_fp8_decode_workspace_bytes(2, 8, 2, 1, 4096, 128, 256) == 4 * 2 * 2 * -(-4096 // 1024) * 4 * 130
    assert fa.attn_fp8_decode_workspace_bytes(2, 8, 3, 1, 4096, 128) == 0


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError, match="device tensor"):
        fa.quantize_qkv_fp8(x, x, x, scale_block=64)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        fa.load_library(str(tmp_path / "missing.so"))
