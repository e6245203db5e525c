"""Exact attention in float64, and the error bars of the FP8 path around it
(oracle; test infrastructure only).

[P2] "Fused attention kernel", Overview: attention is the softmax of the
scaled scores applied to V; the fused kernel visits the keys block by block
and keeps, per query, the largest score seen and the sum of exponentials
against it, rescaling what it has accumulated whenever that maximum grows, so
its result is the plain definition up to rounding order.  Implementation
sketch: the same loop written out, with the output divided by the row sum at
the end and the log-sum-exp returned beside it.  The card's notes on the
paper's listings fix two details: the old state is scaled by the exponential
of (old maximum - new maximum), and the last key block is scored too.

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

from . import e4m3, fastexp, mfma_fp8
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


# ---------------------------------------------------------------------------
# E1 with error bars.  The FP8 path computes E1 (the attention of the
# quantised inputs) with three departures that the pages fix or leave open,
# each bounded here from E1's own quantities (scores, weights, codes,
# descales), never from a kernel's blocking:
#   * P is rounded to e4m3 before its product with V (reading C12; the pages
#     do not model it).  A probability P in e4m3 moves by at most 2^-4 P
#     (normal range, P >= 2^-6) or min(P, 2^-10) (subnormal range), in units
#     where the row's largest P is at least 1 (P carries no V factor: V's
#     power-of-two scale is applied to V).  So |dO_id| <= sum_j b_ij |v_jd|
#     with b_ij = 2^-4 w_ij where w_ij l_i >= 2^-6, else min(w_ij, 2^-10 / l_i),
#     l_i the row sum against the row maximum (l_i >= 1).
#   * The matrix cores sum the e4m3 products with the truncation of
#     ``mfma_fp8``: each score moves by at most delta_ij (natural units);
#     a row whose scores all move by at most D_i has its log-sum-exp moved by
#     at most D_i and every weight scaled by a factor within exp(+-2 D_i), so
#     |dO_id| <= (exp(2 D_i) - 1) sum_j w_ij |v_jd - O_id|.
#   * Optionally Schraudolph's exponential (relative error within
#     [EPS_LO, EPS_HI] per probability, the row sum built from the same
#     values): weights move by a factor within (1 + ETA)^+-1 and the LSE by
#     at most LSE_SCHRAUDOLPH.
# The maximum-error bar of an element is the larger of the target 2e-2 and
# the P-rounding bound, plus the accumulation bound and half a BF16 ulp (the
# output's own rounding).  For the RMS error, P's rounding errors are modelled
# as independent and uniform within their bounds (``sigma``): the RMS bar is
# the larger of the target 2e-3 and twice that model, plus the RMS of the
# accumulation bound.
# ---------------------------------------------------------------------------

EPS_LO = 2.0 ** -fastexp.SIGMA - 1.0 - 2.0 ** -16
EPS_HI = (1.0 / math.log(2.0)) * 2.0 ** (1.0 - 1.0 / math.log(2.0) - fastexp.SIGMA) - 1.0 + 2.0 ** -16
ETA = (1.0 + EPS_HI) / (1.0 + EPS_LO) - 1.0
LSE_SCHRAUDOLPH = max(-math.log1p(EPS_LO), math.log1p(EPS_HI))


def _schraudolph_rel_rms():
    """RMS of Schraudolph's relative error about its mean, over a uniform
    fractional part of the exponent (the part that varies from key to key)."""
    f = (np.arange(1 << 16) + 0.5) / (1 << 16)
    r = fastexp.schraudolph_exp2(f) / np.exp2(f) - 1.0
    return float(np.std(r))


RHO_SCHRAUDOLPH = _schraudolph_rel_rms()


def _per_element(ds, n, d):
    """Descales of n rows as [n, d]: from [n] (one per row) or [n, d / g] (one per g channels)."""
    ds = np.asarray(ds, dtype=np.float64)
    if ds.ndim == 1:
        return np.broadcast_to(ds[:, None], (n, d))
    return np.repeat(ds, d // ds.shape[1], axis=1)


def e1_rows_with_bars(q8r, dq, k8, dk, v8, dv, q_pos, causal, scale, exp2, accumulation):
    """E1 and its bars for R query rows of one sequence against its N keys.

    q8r [R, D], k8 / v8 [N, D] codes; dq [R], dk / dv [N] the descale of each
    row's block, or [R, D / g] / [N, D / g] with one descale per g channels;
    q_pos [R] the query positions (causal: key j is visible iff j <= q_pos).
    Returns O [R, D], LSE [R], bmax [R, D], sigma [R, D], lse_bar [R]
    (what is added to the relative LSE target), acc_bar [R, D].
    """
    R, D = np.shape(q8r)
    N = np.shape(k8)[0]
    dqe, dke, dve = _per_element(dq, R, D), _per_element(dk, N, D), _per_element(dv, N, D)
    qv = e4m3.decode(q8r) * dqe
    kv = e4m3.decode(k8) * dke
    v8v = e4m3.decode(v8)
    vv = v8v * dve
    s = (qv @ kv.T) * scale
    vis = np.ones(s.shape, dtype=bool)
    if causal:
        vis = np.arange(k8.shape[0])[None, :] <= np.asarray(q_pos)[:, None]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    p = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    w = p / l[:, None]
    o = w @ vv
    lse = m + np.log(l)
    wabs = w @ np.abs(vv)
    # sum_j w_ij |v_jd - O_id|, row by row
    wdev = np.empty_like(o)
    for i in range(o.shape[0]):
        wdev[i] = w[i] @ np.abs(vv - o[i])
    # accumulation of the scores by the matrix cores: per score a bound on its
    # movement (the pinned truncation of ``mfma_fp8``, its combination step,
    # and the float32 rounding of the scaled score), then the weighted
    # perturbation of the softmax: with a_j = exp(|delta_j|) - 1 and
    # zeta = sum_j w_j a_j, every weight moves by at most w_j (a_j + zeta) / (1 - zeta)
    # and the LSE by at most -ln(1 - zeta)
    if accumulation:
        # truncation per block of channels that share one descale (the
        # matrix core's groups of 8 never straddle one), in dequantised units
        g = D if np.ndim(dq) == 1 else D // np.shape(dq)[1]
        qc, kc = e4m3.decode(q8r), e4m3.decode(k8)
        d_deq = np.zeros((R, N))
        for c0 in range(0, D, g):
            cs = slice(c0, c0 + g)
            cut = np.abs(mfma_fp8.scores(q8r[:, cs], k8[:, cs]) - qc[:, cs] @ kc[:, cs].T)
            d_deq += cut * np.outer(dqe[:, c0], dke[:, c0])
        # the combination step: FINAL_ULPS float32 ulps of sum |q_c k_c| per
        # instruction, at the scale the products carry (x2: a descale that is
        # not a power of two can put that sum one binade higher)
        abs_deq = np.abs(qv) @ np.abs(kv).T
        ninst = D // mfma_fp8.KBLOCK
        delta = (d_deq + 2.0 * ninst * mfma_fp8.FINAL_ULPS * mfma_fp8.ulp32(abs_deq)) * scale
        delta = delta + 2.0 ** -21 * (np.abs(np.where(vis, s, 0.0)) + np.abs(m)[:, None])
        a = np.where(vis, np.expm1(delta), 0.0)
        zeta = np.sum(w * a, axis=1)
        if np.any(zeta >= 0.5):
            raise ValueError("accumulation error too large for the perturbation bound")
        acc_bar = np.empty_like(o)
        for i in range(o.shape[0]):
            acc_bar[i] = (w[i] * (a[i] + zeta[i])) @ np.abs(vv - o[i]) / (1.0 - zeta[i])
        grow = (1.0 + a.max(axis=1) + zeta) / (1.0 - zeta)
        lse_acc = -np.log1p(-zeta)
    else:
        acc_bar = np.zeros_like(o)
        grow = np.ones(len(m))
        lse_acc = np.zeros(len(m))
    # P's rounding per key, in weight units (P = w l in units where the row
    # maximum is 1, l >= 1): at most 2^-4 P where P is in e4m3's normal range
    # (P >= 2^-6), else at most the smaller of P itself and half the
    # smallest subnormal 2^-10.  A key normal in these units is normal in any
    # larger ones, and below 2^-6 the smaller of the two covers either range.
    pw = w * l[:, None]
    b = np.where(pw >= 2.0 ** -6, 2.0 ** -4 * w, np.minimum(w, 2.0 ** -10 / l[:, None]))
    absvv = np.abs(vv)
    pround = b @ absvv
    var = ((b * b) @ (vv * vv)) / 3.0
    lse_bar = lse_acc.copy()
    if exp2 == "exact":
        pbar = pround
    elif exp2 == "schraudolph":
        pbar = ETA * wdev + pround * (1.0 + ETA)
        dev2 = np.empty_like(o)
        for i in range(o.shape[0]):
            dev2[i] = (w[i] * w[i]) @ (vv - o[i]) ** 2
        var = var + RHO_SCHRAUDOLPH ** 2 * dev2
        lse_bar = lse_bar + LSE_SCHRAUDOLPH
    else:
        raise ValueError("exp2 must be 'exact' or 'schraudolph'")
    return o, lse, pbar * grow[:, None], np.sqrt(var), lse_bar, acc_bar


def emulated_fp8_attention_bars(q8, k8, v8, q_descale, k_descale, v_descale, scale_block, hadamard, causal,
                                rows=None, exp2="exact", accumulation=True, row_chunk=256):
    """E1 (``emulated_fp8_attention``) with the error bars of the FP8 path.

    Returns a dict with O, LSE (E1), and per element / row: ``pbar`` (bound on
    what P's e4m3 rounding, and Schraudolph's exponential if asked, move O),
    ``sigma`` (RMS model of that movement), ``acc_bar`` (bound on what the
    matrix cores' accumulation moves O), ``lse_bar`` (bound on the LSE
    movement beyond the relative target).
    """
    d = np.shape(q8)[-1]
    n = np.shape(q8)[-2]
    lead = np.shape(q8)[:-2]
    scale = 1.0 / math.sqrt(d) / (d if hadamard else 1)
    row_idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    tok_blk = np.arange(n) // scale_block
    out = {k: np.empty(lead + (len(row_idx), d)) for k in ("o", "pbar", "sigma", "acc_bar")}
    out.update({k: np.empty(lead + (len(row_idx),)) for k in ("lse", "lse_bar")})
    for idx in np.ndindex(*lead):
        qd = np.asarray(q_descale[idx], dtype=np.float64)
        kd = np.asarray(k_descale[idx], dtype=np.float64)
        vd = np.asarray(v_descale[idx], dtype=np.float64)
        for c0 in range(0, len(row_idx), row_chunk):
            ri = row_idx[c0:c0 + row_chunk]
            res = e1_rows_with_bars(q8[idx][ri], qd[ri // scale_block], k8[idx], kd[tok_blk], v8[idx],
                                     vd[tok_blk], ri, causal, scale, exp2, accumulation)
            sl = idx + (slice(c0, c0 + len(ri)),)
            for key, val in zip(("o", "lse", "pbar", "sigma", "lse_bar", "acc_bar"), res):
                out[key][sl] = val
    return out


def online_attention_fp64(q, k, v, causal, scale, block_c):
    """Blockwise attention of one head merged by log-sum-exp, float64.

    Each key block of ``block_c`` keys (the last may be short) is reduced on
    its own to (its row maxima, its row sums against them, its unnormalised
    partial output); the blocks are then combined left to right, each
    combination rescaling the side whose maximum is smaller by the exponential
    of the difference.  This is the fused loop's invariant written as a merge
    of independent partial results ("Fused attention kernel", Overview and
    Implementation sketch: the running maximum and sum make the blockwise
    result exact).  Used only to pin ``attention_fp64`` (they must agree).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    qi = np.arange(n)
    parts = []
    for j0 in range(0, k.shape[0], block_c):
        s = (q @ k[j0:j0 + block_c].T) * scale
        if causal:
            kidx = np.arange(j0, j0 + s.shape[1])
            s = np.where(kidx[None, :] <= qi[:, None], s, -np.inf)
        bmax = s.max(axis=1)
        seen = np.isfinite(bmax)                  # rows with a visible key in this block
        e = np.exp(s - np.where(seen, bmax, 0.0)[:, None])
        e[~seen] = 0.0
        parts.append((bmax, e.sum(axis=1), e @ v[j0:j0 + block_c]))
    big, tot, acc = parts[0]
    for bmax, bsum, bout in parts[1:]:
        new = np.maximum(big, bmax)
        ref = np.where(np.isfinite(new), new, 0.0)
        wa = np.where(np.isfinite(big), np.exp(big - ref), 0.0)
        wb = np.where(np.isfinite(bmax), np.exp(bmax - ref), 0.0)
        tot = wa * tot + wb * bsum
        acc = wa[:, None] * acc + wb[:, None] * bout
        big = new
    return acc / tot[:, None], big + np.log(tot)


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


def emulated_fp8_attention_tiled(q8, k8, v8, q_descale, k_descale, v_descale, scale_block, hadamard,
                                 causal, rows=None, tau=8.8, quantize_p=True, bf16_output=True, block_c=64,
                                 exp2="exact", lift=2.0):
    """E2 (a diagnostic, not the contract): the running-softmax loop over key
    blocks with P re-quantised to e4m3, in the FP8 kernel's blocking.

    The pages fix the loop (Implementation sketch) and that the matrix products
    run on 8-bit inputs; they are silent on the precision and scale of P.
    Readings taken here (the FP8 kernel follows them):
      * the loop visits key blocks of ``block_c`` keys (64 in the kernel),
        which must divide ``scale_block``; scores in log2 units:
        t = s * dq_i * dk_j * log2(e) / sqrt(d) (/ d if rotated), s the exact
        dot product of the decoded codes, dk_j the descale of key block j;
      * a reference m is kept per query; it moves only when a block's max
        exceeds m by more than ``tau``, and then to ``lift`` (a whole number)
        below that max, so the key that moved it has P = 2^lift exactly; with
        tau = lift = 0 this is the sketch's running max;
      * P = e4m3(2^(t - m)) <= 2^tau enters the product with V, whose
        (power-of-two) block scale multiplies V itself (the matrix core
        applies it); the old partial output is multiplied by 2^(m_old - m_new)
        when m moves (the sketch's exp(old max - new max));
      * l sums the unquantised 2^(t - m); O = O_acc / l;
        LSE = ln 2 * (m + log2 l), the natural log-sum-exp of the scaled scores;
      * O is delivered in BF16 ([P1] "How it gets verified": BF16 output),
        rounded to nearest even (``bf16_output``); LSE stays float64.
    Arithmetic is float64 apart from the e4m3 rounding of P and the final BF16
    rounding of O.  With ``quantize_p=False, bf16_output=False`` the result
    equals E1 up to float64 rounding.

    ``exp2="schraudolph"`` replaces the probabilities' exponential by
    Schraudolph's bit-level approximation (``fastexp.schraudolph_exp2``) of
    t - m, as the kernel's option does: P = e4m3(S(t - m)) and l sums
    S(t - m).  The rescale 2^(m_old - m_new) stays exact.

    Descales [..., nblk, D / g] (one per block and g channels, the 32-channel
    MX form) scale each channel of Q and K before the dot product and each
    channel of V in the product with P.
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
    grouped = kd.ndim == len(lead) + 2
    for idx in np.ndindex(*lead):
        qh, kh, vh = q[idx][row_idx], k[idx], v[idx]
        qdr = qd[idx][row_idx // scale_block]
        if grouped:
            g = d // kd.shape[-1]
            qh = qh * np.repeat(qdr, g, axis=1)
            qdr = np.ones(len(row_idx))
        m = np.full(len(row_idx), -np.inf)
        l = np.zeros(len(row_idx))
        acc = np.zeros((len(row_idx), d))
        for j in range(nkb):
            k0, k1 = j * block_c, min(n, (j + 1) * block_c)
            sb = k0 // scale_block
            if grouped:
                s = qh @ (kh[k0:k1] * np.repeat(kd[idx][sb], g)[None, :]).T
                t = s * (qdr * score_scale)[:, None]
                vs = vh[k0:k1] * np.repeat(vd[idx][sb], g)[None, :]
            else:
                s = qh @ kh[k0:k1].T
                t = s * (qdr * kd[idx][sb] * score_scale)[:, None]
                vs = vh[k0:k1] * vd[idx][sb]
            if causal:
                t = np.where(np.arange(k0, k1)[None, :] <= row_idx[:, None], t, -np.inf)
            tmax = t.max(axis=1)
            upd = tmax > m + tau
            m_new = np.where(upd, tmax - lift, m)
            alpha = np.where(upd, np.exp2(np.where(np.isfinite(m), m - m_new, -np.inf)), 1.0)
            m = m_new
            ok = np.isfinite(m)
            arg = t - np.where(ok, m, 0.0)[:, None]
            pu = np.exp2(arg) if exp2 == "exact" else fastexp.schraudolph_exp2(arg)
            pu[~ok] = 0.0
            pq = e4m3.decode(e4m3.encode(pu)) if quantize_p else pu
            l = alpha * l + pu.sum(axis=1)
            acc = alpha[:, None] * acc + pq @ vs
        o_all[idx] = acc / l[:, None]
        lse_all[idx] = math.log(2.0) * (m + np.log2(l))
    if bf16_output:
        o_all = round_to_bf16(o_all)
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
