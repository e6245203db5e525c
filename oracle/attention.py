"""Exact attention in float64 and the running-softmax loop (oracle; test infrastructure only).

[P2] "Fused attention kernel", Overview: attention is softmax(Q K^T) V; a fused
kernel reaches the same result block by block with a running row maximum and
row sum, so the fused loop is exact up to rounding order.  Implementation
sketch: per key block, s = q k_j^T, m_new = max(m, rowmax s),
alpha = exp(m - m_new), p = exp(s - m_new), l = alpha l + rowsum p,
o = alpha o + p v_j; at the end o / l and lse = m + log l.  The card scores
every key block (its note on the printed loop bound of the paper's Algorithm 2)
and rescales the output by exp(old max - new max) (its note on Algorithm 1).

Readings taken here (the pages leave them open):
  * softmax scale 1/sqrt(d) on the scores (the sketch prints none);
  * LSE is the natural log of sum_j exp(scaled score);
  * causal (query and key sequences of equal length): key j is visible to
    query i iff j <= i;
  * the reference precision is float64 ([P2] Variants / 8-bit forward pass
    compares against FP64; [P1] "How it gets verified" says 32-bit; float64 is
    the stricter of the two).
"""

import math

import numpy as np

from . import e4m3, fastexp
from .quantize import dequantize


def _rows_attention(q_rows, row_idx, k, v, causal, scale):
    """Attention for the given query rows of one head; float64 in and out."""
    s = (q_rows @ k.T) * scale
    if causal:
        key_idx = np.arange(k.shape[0])
        s = np.where(key_idx[None, :] <= row_idx[:, None], s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]
    return o, m + np.log(l)


def attention_fp64(q, k, v, causal, scale, rows=None, row_chunk=512):
    """softmax(scale * Q K^T [+ causal mask]) V and its log-sum-exp, in float64.

    q, k, v: arrays [..., N, d] (any float type, upcast exactly).  ``rows``
    optionally restricts the queries to those row indices (same for every
    leading index).  Returns (O [..., R, d], LSE [..., R]) with R = N or len(rows).
    The N x N score matrix is never held whole: queries go in chunks.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape[-2], q.shape[-1]
    lead = q.shape[:-2]
    row_idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty(lead + (len(row_idx), d), dtype=np.float64)
    lse = np.empty(lead + (len(row_idx),), dtype=np.float64)
    for idx in np.ndindex(*lead):
        qh, kh, vh = q[idx], k[idx], v[idx]
        for c0 in range(0, len(row_idx), row_chunk):
            ri = row_idx[c0:c0 + row_chunk]
            oc, lc = _rows_attention(qh[ri], ri, kh, vh, causal, scale)
            o[idx + (slice(c0, c0 + len(ri)),)] = oc
            lse[idx + (slice(c0, c0 + len(ri)),)] = lc
    return o, lse


def reference_attention(q, k, v, causal, rows=None):
    """R: exact attention of the float32 inputs in float64 with scale 1/sqrt(d)."""
    d = np.shape(q)[-1]
    return attention_fp64(q, k, v, causal, 1.0 / math.sqrt(d), rows=rows)


def emulated_fp8_attention(q8, k8, v8, q_descale, k_descale, v_descale,
                           scale_block, hadamard, causal, rows=None):
    """E1: exact float64 attention of the dequantised FP8 inputs.

    Q^ = e4m3(q8) * descale_q per block (likewise K^, V^).  With the rotation
    on, Q^ K^^T = d * (Q K^T) up to quantisation error, because the sign
    diagonal and the unnormalised Hadamard matrix satisfy (S H)(S H)^T = d I;
    so the score scale is 1/(sqrt(d) * d).  P is not quantised here: this is
    attention of the quantised inputs, the quantity the FP8 kernel approximates.
    """
    d = np.shape(q8)[-1]
    qh = dequantize(q8, q_descale, scale_block)
    kh = dequantize(k8, k_descale, scale_block)
    vh = dequantize(v8, v_descale, scale_block)
    scale = 1.0 / math.sqrt(d)
    if hadamard:
        scale /= d
    return attention_fp64(qh, kh, vh, causal, scale, rows=rows)


def online_attention_fp64(q, k, v, causal, scale, block_c):
    """The sketch's running-softmax loop for one head, float64, key blocks of ``block_c``.

    Scores every key block including a short last one; rescales the old state
    by exp(m_old - m_new).  Used only to pin ``attention_fp64`` (they must agree).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    nk = k.shape[0]
    o = np.zeros((n, d))
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    qi = np.arange(n)
    for j0 in range(0, nk, block_c):
        kj = k[j0:j0 + block_c]
        vj = v[j0:j0 + block_c]
        s = (q @ kj.T) * scale
        if causal:
            kidx = np.arange(j0, j0 + kj.shape[0])
            s = np.where(kidx[None, :] <= qi[:, None], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        # a row with no visible key yet keeps m = -inf; use 0 as its exp reference
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(np.where(np.isfinite(m), m - ref, -np.inf))
        p = np.exp(s - ref[:, None])
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ vj
        m = m_new
    return o / l[:, None], m + np.log(l)


def brute_force_attention(q, k, v, causal, scale):
    """Explicit Python loops over rows, keys and channels (tiny inputs only)."""
    n, d = len(q), len(q[0])
    nk = len(k)
    o = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        scores = []
        for j in range(nk):
            if causal and j > i:
                continue
            dot = 0.0
            for c in range(d):
                dot += float(q[i][c]) * float(k[j][c])
            scores.append((j, dot * scale))
        mx = max(sc for _, sc in scores)
        total = sum(math.exp(sc - mx) for _, sc in scores)
        for j, sc in scores:
            w = math.exp(sc - mx) / total
            for c in range(d):
                o[i][c] += w * float(v[j][c])
        lse[i] = mx + math.log(total)
    return np.array(o), np.array(lse)


# Relative half-width of the window around an e4m3 rounding midpoint inside
# which a probability evaluated in float32 (its exponent argument carries a
# few float32 roundings of scores up to a few hundred in log2 units, and the
# hardware exponential is within one ulp) can round to either neighbour.
P_TIE_WINDOW = 2.0 ** -14


def e4m3_tie_step(x, window=P_TIE_WINDOW):
    """For x >= 0: the e4m3 spacing at x where x lies within ``window * x`` of
    a rounding midpoint (so either neighbour is a valid rounding at a lower
    precision), else 0."""
    x = np.asarray(x, dtype=np.float64)
    _, fexp = np.frexp(np.where(x > 0, x, 1.0))
    quantum = np.ldexp(1.0, np.maximum(fexp - 1, -6) - 3)
    frac = x / quantum - np.floor(x / quantum)
    near = (x > 0) & (np.abs(frac - 0.5) * quantum <= window * x)
    return np.where(near, quantum, 0.0)


def emulated_fp8_attention_tiled(q8, k8, v8, q_descale, k_descale, v_descale, scale_block, hadamard,
                                 causal, rows=None, tau=8.0, quantize_p=True, bf16_output=True, block_c=64,
                                 exp2="exact", mx=False, tie_slack=False):
    """E2: the running-softmax loop over key blocks with P re-quantised to e4m3.

    The pages fix the loop (Implementation sketch) and that the matrix products
    run on 8-bit inputs; they are silent on the precision and scale of P.
    Reading taken here (the FP8 kernel follows it):
      * the loop visits key blocks of ``block_c`` keys (the sketch's block_c;
        64 in the kernel), which must divide ``scale_block``; scores in log2
        units: t = s * dq_i * dk_j * log2(e) / sqrt(d) (/ d if rotated), where s
        is the exact dot product of the decoded codes and dk_j the descale of
        the scale block holding key block j;
      * a reference max m is kept per query; it moves to a block's max only
        when that max exceeds m by more than ``tau``; with tau = 0 this is the
        sketch's running max (m_new = max(m, rowmax));
      * P entering the product with V is e4m3(2^(t - m) * r_j) with
        r_j = dv_j / dv_ref, dv_ref the largest V descale among the key blocks
        that the query's block can see (all blocks when not causal); so P <= 2^tau;
      * the old partial output is multiplied by 2^(m_old - m_new) when m moves
        (the sketch's exp(old max - new max));
      * l sums the unquantised 2^(t - m); O = dv_ref * O_acc / l;
        LSE = ln 2 * (m + log2 l), the natural log-sum-exp of the scaled scores;
      * O is delivered in BF16 ([P1] "How it gets verified": BF16 output),
        rounded to nearest even (``bf16_output``); LSE stays float64.
    Arithmetic is float64 apart from the e4m3 rounding of P and the final BF16
    rounding of O.  With ``quantize_p=False, bf16_output=False`` the result
    equals E1 up to float64 rounding.

    ``exp2="schraudolph"`` replaces the probabilities' exponential by
    Schraudolph's bit-level approximation (``fastexp.schraudolph_exp2``), taken
    of the whole exponent t - m + log2 r_j, as the kernel's option does:
    P = e4m3(S(t - m + log2 r_j)) and l sums S(t - m + log2 r_j) / r_j.  The
    rescale 2^(m_old - m_new) stays exact.

    ``mx=True`` (power-of-two descales applied to the operands by the matrix
    units): V's block scale multiplies V itself, so P = e4m3(2^(t - m)) carries
    no r_j (dv_ref = 1), and O = O_acc / l with O_acc = sum P (v * dv_j).  With
    power-of-two scales this differs from the default only where e4m3 rounding
    of 2^(t-m) r_j and of 2^(t-m) differ (subnormal P).

    ``tie_slack=True`` also returns, per output element, how far O can move
    when every P whose unrounded value lies within ``P_TIE_WINDOW`` of an
    e4m3 rounding midpoint (``e4m3_tie_step``) rounds to its other neighbour:
    the sum of those rounding steps times |v| (dequantised), carried through
    the rescales and the final normalisation like O itself.  It is the part of
    a lower-precision evaluation's difference that is a valid rounding, not an
    error.  Returns (O, LSE, slack) then.
    """
    if exp2 not in ("exact", "schraudolph"):
        raise ValueError("exp2 must be 'exact' or 'schraudolph'")
    q = e4m3.decode(q8)
    k = e4m3.decode(k8)
    v = e4m3.decode(v8)
    qd = np.asarray(q_descale, dtype=np.float64)
    kd = np.asarray(k_descale, dtype=np.float64)
    vd = np.asarray(v_descale, dtype=np.float64)
    n, d = q.shape[-2], q.shape[-1]
    lead = q.shape[:-2]
    score_scale = math.log2(math.e) / math.sqrt(d) / (d if hadamard else 1)
    row_idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    if scale_block % block_c:
        raise ValueError("block_c must divide scale_block")
    nkb = -(-n // block_c)
    o_all = np.empty(lead + (len(row_idx), d))
    lse_all = np.empty(lead + (len(row_idx),))
    slack_all = np.zeros(lead + (len(row_idx), d))
    for idx in np.ndindex(*lead):
        qh, kh, vh = q[idx][row_idx], k[idx], v[idx]
        qdr = qd[idx][row_idx // scale_block]
        own_blk = row_idx // scale_block
        if mx:
            dv_ref = np.ones(len(row_idx))
        elif causal:
            dv_ref = np.array([vd[idx][:b + 1].max() for b in own_blk])
        else:
            dv_ref = np.full(len(row_idx), vd[idx].max())
        m = np.full(len(row_idx), -np.inf)
        l = np.zeros(len(row_idx))
        acc = np.zeros((len(row_idx), d))
        slk = np.zeros((len(row_idx), d))
        for j in range(nkb):
            k0, k1 = j * block_c, min(n, (j + 1) * block_c)
            sb = k0 // scale_block
            s = qh @ kh[k0:k1].T
            t = s * (qdr * kd[idx][sb] * score_scale)[:, None]
            if causal:
                t = np.where(np.arange(k0, k1)[None, :] <= row_idx[:, None], t, -np.inf)
            tmax = t.max(axis=1)
            upd = tmax > m + tau
            m_new = np.where(upd, tmax, m)
            alpha = np.where(upd, np.exp2(np.where(np.isfinite(m), m - m_new, -np.inf)), 1.0)
            m = m_new
            ok = np.isfinite(m)
            r = np.ones(len(row_idx)) if mx else vd[idx][sb] / dv_ref
            if exp2 == "exact":
                pu = np.exp2(t - np.where(ok, m, 0.0)[:, None])
                pu[~ok] = 0.0
                pq = pu * r[:, None]
            else:
                pq = fastexp.schraudolph_exp2(t - np.where(ok, m, 0.0)[:, None] + np.log2(r)[:, None])
                pq[~ok] = 0.0
                pu = pq / r[:, None]
            vblk = vh[k0:k1] * (vd[idx][sb] if mx else 1.0)
            if tie_slack:
                slk = alpha[:, None] * slk + (e4m3_tie_step(pq) if quantize_p else 0.0 * pq) @ np.abs(vblk)
            if quantize_p:
                pq = e4m3.decode(e4m3.encode(pq))
            l = alpha * l + pu.sum(axis=1)
            acc = alpha[:, None] * acc + pq @ vblk
        o_all[idx] = acc * dv_ref[:, None] / l[:, None]
        lse_all[idx] = math.log(2.0) * (m + np.log2(l))
        if tie_slack:
            slack_all[idx] = slk * dv_ref[:, None] / l[:, None]
    if bf16_output:
        o_all = round_to_bf16(o_all)
    if tie_slack:
        return o_all, lse_all, slack_all
    return o_all, lse_all


def round_to_bf16(x):
    """Nearest bfloat16 value (ties to even) of each float64, returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; the value is
    rounded once from float64 (no intermediate float32 rounding).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, fexp = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(fexp - 1, -126)
    quantum = np.ldexp(1.0, e - 7)
    return np.copysign(np.rint(a / quantum) * quantum, x)
