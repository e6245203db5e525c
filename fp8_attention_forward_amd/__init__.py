"""Python binding of the gfx950 FP8 fused attention forward library (libattn_fp8.so).

A thin ctypes layer with the same names as the C ABI (include/attn_fp8.h).  It
only marshals arguments: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or a call fails, an exception
is raised.

    q8, k8, v8, qd, kd, vd = quantize_qkv_fp8(q, k, v, scale_block=128, hadamard=True, seed=0x5EED)
    o, lse = attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=128, hadamard=True, causal=False)
    o, lse = attn_fp8_fwd(..., exp2="schraudolph")   # Schraudolph's bit-level exponential
    o16, lse16 = attn_bf16_fwd(qb, kb, vb, causal=False)

Packed variable-length documents ([H, T, D] tensors, int32 cu_seqlens on the device):

    q8, k8, v8, qd, kd, vd = quantize_qkv_fp8_varlen(q, k, v, cu_seqlens, scale_block=128)
    o, lse = attn_fp8_fwd_varlen(q8, k8, v8, qd, kd, vd, cu_seqlens, scale_block=128, causal=True)

Decode against an FP8 K/V cache (cache from quantize_qkv_fp8 on the sequences, queries from
quantize_qkv_fp8 on the new tokens; int32 seqlens on the device):

    o, lse = attn_fp8_decode(q8, q_descale, k8, v8, k_descale, v_descale, seqlens, scale_block=128)
"""

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "AttnError", "load_library", "quantize_qkv_fp8", "attn_fp8_fwd", "attn_bf16_fwd",
    "last_error", "abi_version", "EXPORTED_SYMBOLS", "ATTN_OK", "ATTN_EINVAL", "ATTN_EUNSUPPORTED", "ATTN_EHIP",
    "ATTN_FP8_EXP2_SCHRAUDOLPH", "ATTN_FP8_MX", "ATTN_FP8_MX32", "ATTN_FP8_NATURAL_ORDER", "EXP2_MODES", "ORDERS",
    "quantize_qkv_fp8_varlen", "attn_fp8_fwd_varlen", "attn_fp8_varlen_workspace_bytes", "varlen_num_slots",
    "attn_fp8_decode", "attn_fp8_decode_workspace_bytes", "attn_fp8_decode_split", "attn_fp8_decode_noalloc",
    "DECODE_NOALLOC_MAX_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_fp8.so")
ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP = 0, 1, 2, 3
ATTN_FP8_EXP2_SCHRAUDOLPH = 1
ATTN_FP8_MX = 2
ATTN_FP8_NATURAL_ORDER = 4
ATTN_FP8_MX32 = 8
ORDERS = {"longest_first": 0, "natural": ATTN_FP8_NATURAL_ORDER}
EXP2_MODES = {"exact": 0, "schraudolph": ATTN_FP8_EXP2_SCHRAUDOLPH}
EXPORTED_SYMBOLS = ("quantize_qkv_fp8", "quantize_qkv_fp8_opts", "attn_fp8_fwd", "attn_fp8_fwd_opts", "attn_bf16_fwd",
                    "quantize_qkv_fp8_varlen", "attn_fp8_varlen_workspace_bytes", "attn_fp8_fwd_varlen",
                    "attn_fp8_decode_split", "attn_fp8_decode_workspace_bytes", "attn_fp8_decode",
                    "attn_fp8_decode_noalloc",
                    "attn_fp8_last_error", "attn_fp8_abi_version")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def load_library(path=None):
    """Load libattn_fp8.so (built in place by fp8_attention_forward_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} not found: build it with `python -m fp8_attention_forward_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    lib.quantize_qkv_fp8.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, u64, vp, vp, vp, vp, vp, vp, vp]
    lib.quantize_qkv_fp8.restype = i32
    lib.quantize_qkv_fp8_opts.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, u64, ctypes.c_uint,
                                          vp, vp, vp, vp, vp, vp, vp]
    lib.quantize_qkv_fp8_opts.restype = i32
    lib.attn_fp8_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.attn_fp8_fwd.restype = i32
    lib.attn_fp8_fwd_opts.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, ctypes.c_uint,
                                      vp, vp, vp]
    lib.attn_fp8_fwd_opts.restype = i32
    lib.attn_bf16_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.attn_bf16_fwd.restype = i32
    lib.quantize_qkv_fp8_varlen.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, u64, ctypes.c_uint,
                                            vp, vp, vp, vp, vp, vp, vp]
    lib.quantize_qkv_fp8_varlen.restype = i32
    lib.attn_fp8_varlen_workspace_bytes.argtypes = [i32, i32]
    lib.attn_fp8_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fp8_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, ctypes.c_uint,
                                        vp, ctypes.c_size_t, vp, vp, vp]
    lib.attn_fp8_fwd_varlen.restype = i32
    lib.attn_fp8_decode_split.argtypes = [i32, i32, i32, i32]
    lib.attn_fp8_decode_split.restype = i32
    lib.attn_fp8_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.attn_fp8_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fp8_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                    vp, ctypes.c_size_t, vp, vp, vp]
    lib.attn_fp8_decode.restype = i32
    lib.attn_fp8_decode_noalloc.argtypes = [vp] * 7 + [i32] * 10 + [vp] * 3
    lib.attn_fp8_decode_noalloc.restype = i32
    lib.attn_fp8_last_error.argtypes = []
    lib.attn_fp8_last_error.restype = ctypes.c_char_p
    lib.attn_fp8_abi_version.argtypes = []
    lib.attn_fp8_abi_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def last_error():
    return load_library().attn_fp8_last_error().decode()


def abi_version():
    return load_library().attn_fp8_abi_version()


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, last_error())


def _ptr(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shape4(t, name):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, D]")
    return tuple(int(x) for x in t.shape)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def quantize_qkv_fp8(q, k, v, scale_block=128, hadamard=True, seed=0x5EED, out=None, mx=False, mx32=False):
    """Rotate (Q, K) + per-block scale + e4m3 encode; returns (q8, k8, v8, q_descale, k_descale, v_descale).

    mx=True: power-of-two (E8M0) block scales (quantize_qkv_fp8_opts with ATTN_FP8_MX).
    mx32=True: one power-of-two scale per block x 32 channels (ATTN_FP8_MX32); descales [B, H, nblk, D / 32].
    """
    lib = load_library()
    B, H, N, D = _shape4(q, "q")
    if _shape4(k, "k") != (B, H, N, D) or _shape4(v, "v") != (B, H, N, D):
        raise ValueError("q, k, v must have the same shape")
    nb = -(-N // scale_block)
    dshape = (B, H, nb, D // 32) if mx32 else (B, H, nb)
    if out is None:
        dev = q.device
        out = tuple(torch.empty((B, H, N, D), dtype=torch.uint8, device=dev) for _ in range(3)) + \
            tuple(torch.empty(dshape, dtype=torch.float32, device=dev) for _ in range(3))
    q8, k8, v8, qd, kd, vd = out
    for t, nm in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if _shape4(t, nm) != (B, H, N, D):
            raise ValueError(f"{nm} has the wrong shape")
    for t, nm in ((qd, "q_descale"), (kd, "k_descale"), (vd, "v_descale")):
        if tuple(t.shape) != dshape:
            raise ValueError(f"{nm} must be {list(dshape)}")
    head = (_ptr(q, torch.float32, "q"), _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
            B, H, N, D, int(scale_block), int(bool(hadamard)), int(seed) & 0xFFFFFFFFFFFFFFFF)
    tail = (_ptr(q8, torch.uint8, "q8"), _ptr(k8, torch.uint8, "k8"), _ptr(v8, torch.uint8, "v8"),
            _ptr(qd, torch.float32, "q_descale"), _ptr(kd, torch.float32, "k_descale"),
            _ptr(vd, torch.float32, "v_descale"), _stream(q))
    if mx or mx32:
        _check(lib.quantize_qkv_fp8_opts(*head, ATTN_FP8_MX32 if mx32 else ATTN_FP8_MX, *tail))
    else:
        _check(lib.quantize_qkv_fp8(*head, *tail))
    return out


def attn_fp8_fwd(q8, k8, v8, q_descale, k_descale, v_descale, scale_block=128, hadamard=True,
                 causal=False, out=None, exp2="exact", mx=False, mx32=False):
    """FP8 attention forward; returns (o [B,H,N,D] bfloat16, lse [B,H,N] float32).

    exp2: "exact" or "schraudolph" (ATTN_FP8_EXP2_SCHRAUDOLPH: bit-level
    exponentials for the probabilities).  mx=True: power-of-two descales
    applied by the matrix cores (ATTN_FP8_MX); mx32=True: the same per 32
    channels (ATTN_FP8_MX32, descales [B, H, nblk, D / 32]).  Any option goes
    through attn_fp8_fwd_opts, none through attn_fp8_fwd.
    """
    lib = load_library()
    if exp2 not in EXP2_MODES:
        raise ValueError(f"exp2 must be one of {sorted(EXP2_MODES)}")
    B, H, N, D = _shape4(q8, "q8")
    if _shape4(k8, "k8") != (B, H, N, D) or _shape4(v8, "v8") != (B, H, N, D):
        raise ValueError("q8, k8, v8 must have the same shape")
    nb = -(-N // scale_block)
    dshape = (B, H, nb, D // 32) if mx32 else (B, H, nb)
    for t, nm in ((q_descale, "q_descale"), (k_descale, "k_descale"), (v_descale, "v_descale")):
        if tuple(t.shape) != dshape:
            raise ValueError(f"{nm} must be {list(dshape)}")
    if out is None:
        out = (torch.empty((B, H, N, D), dtype=torch.bfloat16, device=q8.device),
               torch.empty((B, H, N), dtype=torch.float32, device=q8.device))
    o, lse = out
    if _shape4(o, "o") != (B, H, N, D) or tuple(lse.shape) != (B, H, N):
        raise ValueError("o / lse have the wrong shape")
    args = (_ptr(q8, torch.uint8, "q8"), _ptr(k8, torch.uint8, "k8"), _ptr(v8, torch.uint8, "v8"),
            _ptr(q_descale, torch.float32, "q_descale"), _ptr(k_descale, torch.float32, "k_descale"),
            _ptr(v_descale, torch.float32, "v_descale"), B, H, N, D, int(scale_block), int(bool(hadamard)),
            int(bool(causal)))
    tail = (_ptr(o, torch.bfloat16, "o"), _ptr(lse, torch.float32, "lse"), _stream(q8))
    flags = EXP2_MODES[exp2] | (ATTN_FP8_MX32 if mx32 else (ATTN_FP8_MX if mx else 0))
    if flags == 0:
        _check(lib.attn_fp8_fwd(*args, *tail))
    else:
        _check(lib.attn_fp8_fwd_opts(*args, flags, *tail))
    return out


def attn_bf16_fwd(q, k, v, causal=False, out=None):
    """BF16 attention forward (the 16-bit yardstick); returns (o bfloat16, lse float32)."""
    lib = load_library()
    B, H, N, D = _shape4(q, "q")
    if _shape4(k, "k") != (B, H, N, D) or _shape4(v, "v") != (B, H, N, D):
        raise ValueError("q, k, v must have the same shape")
    if out is None:
        out = (torch.empty((B, H, N, D), dtype=torch.bfloat16, device=q.device),
               torch.empty((B, H, N), dtype=torch.float32, device=q.device))
    o, lse = out
    _check(lib.attn_bf16_fwd(
        _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"),
        B, H, N, D, int(bool(causal)), _ptr(o, torch.bfloat16, "o"), _ptr(lse, torch.float32, "lse"),
        _stream(q)))
    return out


def _shape3(t, name):
    if t.dim() != 3:
        raise ValueError(f"{name} must be [H, T, D]")
    return tuple(int(x) for x in t.shape)


def _cu(cu_seqlens, T):
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-D tensor of ndoc + 1 entries")
    return _ptr(cu_seqlens, torch.int32, "cu_seqlens"), int(cu_seqlens.numel()) - 1


def varlen_num_slots(T, ndoc, scale_block):
    """Descale entries per head of packed documents: T // scale_block + ndoc."""
    return T // scale_block + ndoc


def attn_fp8_varlen_workspace_bytes(T, ndoc):
    return int(load_library().attn_fp8_varlen_workspace_bytes(int(T), int(ndoc)))


def quantize_qkv_fp8_varlen(q, k, v, cu_seqlens, scale_block=128, hadamard=True, seed=0x5EED, out=None, mx=False):
    """Packed documents: q, k, v float32 [H, T, D], cu_seqlens int32 [ndoc + 1] (device).

    Returns (q8, k8, v8 [H, T, D] uint8, q/k/v_descale [H, T // scale_block + ndoc] float32);
    descale entries that belong to no block are left as allocated.
    """
    lib = load_library()
    H, T, D = _shape3(q, "q")
    if _shape3(k, "k") != (H, T, D) or _shape3(v, "v") != (H, T, D):
        raise ValueError("q, k, v must have the same shape")
    cu, ndoc = _cu(cu_seqlens, T)
    ns = varlen_num_slots(T, ndoc, scale_block)
    if out is None:
        dev = q.device
        out = tuple(torch.empty((H, T, D), dtype=torch.uint8, device=dev) for _ in range(3)) + \
            tuple(torch.empty((H, ns), dtype=torch.float32, device=dev) for _ in range(3))
    q8, k8, v8, qd, kd, vd = out
    for t, nm in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if _shape3(t, nm) != (H, T, D):
            raise ValueError(f"{nm} has the wrong shape")
    for t, nm in ((qd, "q_descale"), (kd, "k_descale"), (vd, "v_descale")):
        if tuple(t.shape) != (H, ns):
            raise ValueError(f"{nm} must be [H, T // scale_block + ndoc]")
    _check(lib.quantize_qkv_fp8_varlen(
        _ptr(q, torch.float32, "q"), _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"), cu, ndoc,
        H, T, D, int(scale_block), int(bool(hadamard)), int(seed) & 0xFFFFFFFFFFFFFFFF, ATTN_FP8_MX if mx else 0,
        _ptr(q8, torch.uint8, "q8"), _ptr(k8, torch.uint8, "k8"), _ptr(v8, torch.uint8, "v8"),
        _ptr(qd, torch.float32, "q_descale"), _ptr(kd, torch.float32, "k_descale"),
        _ptr(vd, torch.float32, "v_descale"), _stream(q)))
    return out


def attn_fp8_fwd_varlen(q8, k8, v8, q_descale, k_descale, v_descale, cu_seqlens, scale_block=128, hadamard=True,
                        causal=False, out=None, exp2="exact", mx=False, order="longest_first", workspace=None):
    """FP8 attention of packed documents; returns (o [H, T, D] bfloat16, lse [H, T] float32).

    order: "longest_first" (default) or "natural" (ATTN_FP8_NATURAL_ORDER).
    workspace: optional uint8 device tensor of at least
    attn_fp8_varlen_workspace_bytes(T, ndoc) bytes (allocated here if None).
    """
    lib = load_library()
    if exp2 not in EXP2_MODES:
        raise ValueError(f"exp2 must be one of {sorted(EXP2_MODES)}")
    if order not in ORDERS:
        raise ValueError(f"order must be one of {sorted(ORDERS)}")
    H, T, D = _shape3(q8, "q8")
    if _shape3(k8, "k8") != (H, T, D) or _shape3(v8, "v8") != (H, T, D):
        raise ValueError("q8, k8, v8 must have the same shape")
    cu, ndoc = _cu(cu_seqlens, T)
    ns = varlen_num_slots(T, ndoc, scale_block)
    for t, nm in ((q_descale, "q_descale"), (k_descale, "k_descale"), (v_descale, "v_descale")):
        if tuple(t.shape) != (H, ns):
            raise ValueError(f"{nm} must be [H, T // scale_block + ndoc]")
    need = attn_fp8_varlen_workspace_bytes(T, ndoc)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q8.device)
    if out is None:
        out = (torch.empty((H, T, D), dtype=torch.bfloat16, device=q8.device),
               torch.empty((H, T), dtype=torch.float32, device=q8.device))
    o, lse = out
    if _shape3(o, "o") != (H, T, D) or tuple(lse.shape) != (H, T):
        raise ValueError("o / lse have the wrong shape")
    flags = EXP2_MODES[exp2] | (ATTN_FP8_MX if mx else 0) | ORDERS[order]
    _check(lib.attn_fp8_fwd_varlen(
        _ptr(q8, torch.uint8, "q8"), _ptr(k8, torch.uint8, "k8"), _ptr(v8, torch.uint8, "v8"),
        _ptr(q_descale, torch.float32, "q_descale"), _ptr(k_descale, torch.float32, "k_descale"),
        _ptr(v_descale, torch.float32, "v_descale"), cu, ndoc, H, T, D, int(scale_block), int(bool(hadamard)),
        int(bool(causal)), flags, _ptr(workspace, torch.uint8, "workspace"), ctypes.c_size_t(workspace.numel()),
        _ptr(o, torch.bfloat16, "o"), _ptr(lse, torch.float32, "lse"), _stream(q8)))
    return out


def attn_fp8_decode_split(B, Hkv, Ncap, split=0):
    return int(load_library().attn_fp8_decode_split(int(B), int(Hkv), int(Ncap), int(split)))


def attn_fp8_decode_workspace_bytes(B, Hq, Hkv, Sq, Ncap, D, split=0):
    return int(load_library().attn_fp8_decode_workspace_bytes(int(B), int(Hq), int(Hkv), int(Sq), int(Ncap), int(D),
                                                              int(split)))


DECODE_NOALLOC_MAX_BYTES = 16 << 20       # ATTN_FP8_DECODE_NOALLOC_MAX_BYTES


def attn_fp8_decode(q8, q_descale, k8, v8, k_descale, v_descale, seqlens, scale_block=128, hadamard=True,
                    causal=True, split=0, out=None, workspace=None):
    """Decode: q8 [B, Hq, Sq, D] uint8 with q_descale [B, Hq] or [B, Hq, 1]; cache k8, v8 [B, Hkv, Ncap, D]
    with descales [B, Hkv, ceil(Ncap / scale_block)]; seqlens int32 [B] (device).

    Returns (o [B, Hq, Sq, D] bfloat16, lse [B, Hq, Sq] float32).  split: 0 = the library's choice (balanced
    per-wave shares of the batch's key tiles up to 512 sequences, fixed ranges above), > 0 = fixed ranges of
    that many keys per wave; workspace: optional uint8 device tensor (allocated here if None).
    """
    lib = load_library()
    B, Hq, Sq, D = _shape4(q8, "q8")
    Bk, Hkv, Ncap, Dk = _shape4(k8, "k8")
    if (Bk, Dk) != (B, D) or _shape4(v8, "v8") != (B, Hkv, Ncap, D):
        raise ValueError("k8 / v8 must be [B, Hkv, Ncap, D] with the queries' B and D")
    if tuple(q_descale.shape) not in ((B, Hq), (B, Hq, 1)):
        raise ValueError("q_descale must be [B, Hq] (or [B, Hq, 1])")
    nb = -(-Ncap // scale_block)
    for t, nm in ((k_descale, "k_descale"), (v_descale, "v_descale")):
        if tuple(t.shape) != (B, Hkv, nb):
            raise ValueError(f"{nm} must be [B, Hkv, ceil(Ncap / scale_block)]")
    if seqlens.dim() != 1 or seqlens.numel() != B:
        raise ValueError("seqlens must be [B]")
    need = attn_fp8_decode_workspace_bytes(B, Hq, Hkv, Sq, Ncap, D, split)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q8.device)
    if out is None:
        out = (torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=q8.device),
               torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device))
    o, lse = out
    if _shape4(o, "o") != (B, Hq, Sq, D) or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("o / lse have the wrong shape")
    _check(lib.attn_fp8_decode(
        _ptr(q8, torch.uint8, "q8"), _ptr(q_descale, torch.float32, "q_descale"), _ptr(k8, torch.uint8, "k8"),
        _ptr(v8, torch.uint8, "v8"), _ptr(k_descale, torch.float32, "k_descale"),
        _ptr(v_descale, torch.float32, "v_descale"), _ptr(seqlens, torch.int32, "seqlens"), B, Hq, Hkv, Sq, Ncap, D,
        int(scale_block), int(bool(hadamard)), int(bool(causal)), int(split), _ptr(workspace, torch.uint8, "workspace"),
        ctypes.c_size_t(workspace.numel()), _ptr(o, torch.bfloat16, "o"), _ptr(lse, torch.float32, "lse"),
        _stream(q8)))
    return out


def attn_fp8_decode_noalloc(q8, q_descale, k8, v8, k_descale, v_descale, seqlens, out, scale_block=128,
                            hadamard=True, causal=True, split=0):
    """attn_fp8_decode with no workspace and no allocation: the partials live in the
    library's per-GPU scratch array (see include/attn_fp8.h).  ``out`` = (o, lse) must be
    given (o [B, Hq, Sq, D] bfloat16, lse [B, Hq, Sq] float32); returns it."""
    lib = load_library()
    B, Hq, Sq, D = _shape4(q8, "q8")
    Bk, Hkv, Ncap, Dk = _shape4(k8, "k8")
    if (Bk, Dk) != (B, D) or _shape4(v8, "v8") != (B, Hkv, Ncap, D):
        raise ValueError("k8 / v8 must be [B, Hkv, Ncap, D] with the queries' B and D")
    if tuple(q_descale.shape) not in ((B, Hq), (B, Hq, 1)):
        raise ValueError("q_descale must be [B, Hq] (or [B, Hq, 1])")
    nb = -(-Ncap // scale_block)
    for t, nm in ((k_descale, "k_descale"), (v_descale, "v_descale")):
        if tuple(t.shape) != (B, Hkv, nb):
            raise ValueError(f"{nm} must be [B, Hkv, ceil(Ncap / scale_block)]")
    if seqlens.dim() != 1 or seqlens.numel() != B:
        raise ValueError("seqlens must be [B]")
    o, lse = out
    if _shape4(o, "o") != (B, Hq, Sq, D) or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("o / lse have the wrong shape")
    _check(lib.attn_fp8_decode_noalloc(
        _ptr(q8, torch.uint8, "q8"), _ptr(q_descale, torch.float32, "q_descale"), _ptr(k8, torch.uint8, "k8"),
        _ptr(v8, torch.uint8, "v8"), _ptr(k_descale, torch.float32, "k_descale"),
        _ptr(v_descale, torch.float32, "v_descale"), _ptr(seqlens, torch.int32, "seqlens"), B, Hq, Hkv, Sq, Ncap, D,
        int(scale_block), int(bool(hadamard)), int(bool(causal)), int(split), _ptr(o, torch.bfloat16, "o"),
        _ptr(lse, torch.float32, "lse"), _stream(q8)))
    return out
