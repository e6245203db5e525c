"""Decode over an FP8 K/V cache (oracle; test infrastructure only).

[P1] "FP8 attention that keeps FlashAttention-3 throughput at BF16-level
accuracy", Realistic applications: keeping K and V in FP8 relieves the
bandwidth of the KV cache.  A decode step is the attention of a few new
queries against the long cached K and V of their sequence; with e4m3 codes
the cache moves one byte per element.

The pages give no decode algorithm.  Readings taken here:
  * the cache is what ``quantize.quantize_qkv`` writes for the whole
    sequence: codes [B][Hkv][Ncap][D] and descales [B][Hkv][ceil(Ncap / SB)];
    sequence b uses its first L_b tokens (the new tokens included);
  * queries: the Sq newest tokens, codes [B][Hq][Sq][D] with one descale per
    (b, head) (their single block, Sq <= SB), rotated like K when the
    rotation is on.  Query head h reads K/V head h // G with G = Hq / Hkv
    (grouped queries; G = 1 is plain multi-head attention);
  * query i sits at position L_b - Sq + i.  Causal: it sees the keys up to
    its position; otherwise all L_b keys;
  * the keys are split into ranges of ``split`` consecutive keys (a multiple
    of the 64-key tile).  Each range runs the E2 loop of ``attention`` on its
    own: tiles of 64 keys, the lazy reference (threshold tau, moved to
    ``lift`` below the block maximum), P = e4m3(2^(t - m)) against V scaled
    by its power-of-two block descale, l summing the unrounded 2^(t - m); it
    yields (m, l, O^ = sum P v).  The ranges merge
    exactly: M = max m, w = 2^(m - M), O = sum w O^ / sum w l,
    LSE = ln 2 (M + log2 sum w l).  Without the rounding of P, the split
    changes nothing but rounding order;
  * O is rounded to BF16 at the end; LSE stays float64.
"""

import math

import numpy as np

from . import e4m3
from .attention import e1_rows_with_bars, round_to_bf16

TILE = 64


def emulated_fp8_decode(q8, q_descale, k8, v8, k_descale, v_descale, seqlens, scale_block, hadamard, causal,
                        split, tau=8.8, quantize_p=True, bf16_output=True, lift=2.0):
    """Decode of [B][Hq][Sq][D] query codes against the FP8 cache, in the
    kernel's key ranges (a diagnostic; the contract is E1,
    ``emulated_fp8_decode_bars``).  Returns (O [B][Hq][Sq][D], LSE [B][Hq][Sq])
    in float64 (O rounded to BF16 values unless ``bf16_output`` is False)."""
    if split % TILE or scale_block % TILE:
        raise ValueError("split and scale_block must be multiples of 64")
    B, Hq, Sq, D = np.shape(q8)
    Hkv = np.shape(k8)[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    qv = e4m3.decode(q8)
    kv = e4m3.decode(k8)
    vv = e4m3.decode(v8)
    qd = np.asarray(q_descale, dtype=np.float64)
    kd = np.asarray(k_descale, dtype=np.float64)
    vd = np.asarray(v_descale, dtype=np.float64)
    score_scale = math.log2(math.e) / math.sqrt(D) / (D if hadamard else 1)
    o = np.zeros((B, Hq, Sq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        L = int(seqlens[b])
        if not Sq <= L <= np.shape(k8)[2]:
            raise ValueError("need Sq <= L_b <= Ncap")
        pos = L - Sq + np.arange(Sq)
        for h in range(Hq):
            g = h // G
            q = qv[b, h]
            c = qd[b, h, 0] * score_scale
            parts = []
            for r0 in range(0, L, split):
                r1 = min(L, r0 + split)
                m = np.full(Sq, -np.inf)
                l = np.zeros(Sq)
                acc = np.zeros((Sq, D))
                for k0 in range(r0, r1, TILE):
                    k1 = min(r1, k0 + TILE)
                    blk = k0 // scale_block
                    t = (q @ kv[b, g, k0:k1].T) * (c * kd[b, g, blk])
                    if causal:
                        t = np.where(np.arange(k0, k1)[None, :] <= pos[:, None], t, -np.inf)
                    tmax = t.max(axis=1)
                    upd = tmax > m + tau
                    m_new = np.where(upd, tmax - lift, m)
                    with np.errstate(invalid="ignore"):      # (-inf) - (-inf) in the branch not taken
                        alpha = np.where(upd, np.exp2(np.where(np.isfinite(m), m - m_new, -np.inf)), 1.0)
                    m = m_new
                    ok = np.isfinite(m)
                    pu = np.exp2(t - np.where(ok, m, 0.0)[:, None])
                    pu[~ok] = 0.0
                    pq = e4m3.decode(e4m3.encode(pu)) if quantize_p else pu
                    l = alpha * l + pu.sum(axis=1)
                    acc = alpha[:, None] * acc + pq @ (vv[b, g, k0:k1] * vd[b, g, blk])
                parts.append((m, l, acc))
            M = np.max([p[0] for p in parts], axis=0)
            w = [np.where(np.isfinite(p[0]), np.exp2(p[0] - M), 0.0) for p in parts]
            lt = sum(wi * p[1] for wi, p in zip(w, parts))
            ot = sum(wi[:, None] * p[2] for wi, p in zip(w, parts))
            o[b, h] = ot / lt[:, None]
            lse[b, h] = math.log(2.0) * (M + np.log2(lt))
    if bf16_output:
        o = round_to_bf16(o)
    return o, lse


def emulated_fp8_decode_bars(q8, q_descale, k8, v8, k_descale, v_descale, seqlens, scale_block, hadamard, causal,
                             exp2="exact"):
    """E1 of the decode step, with the FP8 error bars of
    ``attention.emulated_fp8_attention_bars``: for every (sequence, query head)
    the exact float64 attention of its Sq dequantised query rows (one descale)
    against the dequantised first L_b cache rows of its K/V head, query i at
    position L_b - Sq + i.  No split: the ranges of the kernel merge exactly.
    Returns a dict with O and the bars [B, Hq, Sq, D], LSE and its bar [B, Hq, Sq]."""
    B, Hq, Sq, D = np.shape(q8)
    Hkv = np.shape(k8)[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) / (D if hadamard else 1)
    out = {key: np.empty((B, Hq, Sq, D)) for key in ("o", "pbar", "sigma", "acc_bar")}
    out.update({key: np.empty((B, Hq, Sq)) for key in ("lse", "lse_bar")})
    for b in range(B):
        L = int(seqlens[b])
        if not Sq <= L <= np.shape(k8)[2]:
            raise ValueError("need Sq <= L_b <= Ncap")
        blk = np.arange(L) // scale_block
        for h in range(Hq):
            g = h // G
            kd = np.asarray(k_descale[b, g], dtype=np.float64)[blk]
            vd = np.asarray(v_descale[b, g], dtype=np.float64)[blk]
            qd = np.full(Sq, float(q_descale[b, h, 0]))
            res = e1_rows_with_bars(q8[b, h], qd, k8[b, g, :L], kd, v8[b, g, :L], vd, L - Sq + np.arange(Sq),
                                    causal, scale, exp2, True)
            for key, val in zip(("o", "lse", "pbar", "sigma", "lse_bar", "acc_bar"), res):
                out[key][b, h] = val
    return out
