"""Pins of the packed-document oracle (oracle.varlen): the descale slot layout
worked out by hand and by brute force, document-local block maxima against an
explicit loop (and an independent Hadamard matrix), attention against masked
softmax over the whole packed sequence, slot reads against a per-token lookup,
no leakage between documents, the one-document case, and the work items."""

import math

import numpy as np
import pytest
import scipy.linalg

from oracle import attention, e4m3, varlen
from oracle.philox import sign_vector


def _random_cu(rng, T, ndoc, zeros=True):
    cuts = np.sort(rng.integers(0, T + 1, size=ndoc - 1))
    cu = np.concatenate([[0], cuts, [T]]).astype(np.int64)
    if not zeros:
        assert np.all(np.diff(cu) > 0)
    return cu


def test_slot_layout_worked_example():
    # blocks of 128: doc 0 = 300 tokens -> slots 0, 1, 2; doc 1 empty; doc 2 = 128
    # tokens from 300 -> 300 // 128 + 2 = 4; doc 3 = 572 tokens from 428 ->
    # 428 // 128 + 3 = 6 .. 10; 1000 // 128 + 4 = 11 slots; 3 and 5 unused
    cu = [0, 300, 300, 428, 1000]
    assert [varlen.first_slot(cu, d, 128) for d in range(4)] == [0, 3, 4, 6]
    assert varlen.num_slots(1000, 4, 128) == 11
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 1000, 64)).astype(np.float32)
    out = varlen.quantize_qkv_varlen(x, x, x, cu, 128, False, 1)
    used = {0, 1, 2, 4, 6, 7, 8, 9, 10}
    for s in range(11):
        assert np.isfinite(out[3][0, s]) == (s in used)


@pytest.mark.parametrize("sb", [64, 128])
def test_slots_are_distinct_and_fit(sb):
    rng = np.random.default_rng(sb)
    for trial in range(300):
        T = int(rng.integers(1, 3000))
        ndoc = int(rng.integers(1, 40))
        cu = _random_cu(rng, T, ndoc)
        seen = set()
        for d in range(ndoc):
            nb = -(-(int(cu[d + 1]) - int(cu[d])) // sb)
            for b in range(nb):
                s = varlen.first_slot(cu, d, sb) + b
                assert 0 <= s < varlen.num_slots(T, ndoc, sb)
                assert s not in seen
                seen.add(s)


def _docs_with_spikes(rng, H, cu, D):
    """Each document at its own magnitude, with a spike on its first and last token."""
    T = int(cu[-1])
    x = rng.standard_normal((H, T, D)).astype(np.float32)
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        if a == b:
            continue
        x[:, a:b] *= np.float32(10.0 ** ((d % 5) - 2))
        x[:, a, 0] = np.float32(50.0 * 10.0 ** ((d % 5) - 2))
        x[:, b - 1, 1] = np.float32(-70.0 * 10.0 ** ((d % 5) - 2))
    return x


@pytest.mark.parametrize("sb", [64, 128])
def test_block_maxima_are_document_local(sb):
    rng = np.random.default_rng(3)
    H, D, T = 2, 64, 1111
    cu = np.array([0, 5, 5, 200, 201, 700, 1111])
    q = _docs_with_spikes(rng, H, cu, D)
    k = _docs_with_spikes(rng, H, cu, D)
    v = _docs_with_spikes(rng, H, cu, D)
    out = varlen.quantize_qkv_varlen(q, k, v, cu, sb, False, 7)
    for i, x in enumerate((q, k, v)):
        desc = out[3 + i]
        for h in range(H):
            for d in range(len(cu) - 1):
                a, b = int(cu[d]), int(cu[d + 1])
                s0 = varlen.first_slot(cu, d, sb)
                for blk, r0 in enumerate(range(a, b, sb)):
                    amax = np.float32(0.0)
                    for r in range(r0, min(b, r0 + sb)):
                        amax = max(amax, np.abs(x[h, r]).max())
                    if i < 2:
                        assert desc[h, s0 + blk] == np.float32(amax) / np.float32(448.0)
                    else:                    # V: the smallest power of two 2^e with amax <= 448 * 2^e
                        e = np.log2(desc[h, s0 + blk])
                        assert e == np.round(e) and amax <= 448.0 * 2.0 ** e and amax > 224.0 * 2.0 ** e
        # codes: each element at its own block's scale (nonzero elements decode near x)
        dec = e4m3.decode(out[i])
        for h in range(H):
            for d in range(len(cu) - 1):
                a, b = int(cu[d]), int(cu[d + 1])
                s0 = varlen.first_slot(cu, d, sb)
                for blk, r0 in enumerate(range(a, b, sb)):
                    r1 = min(b, r0 + sb)
                    y = dec[h, r0:r1] * desc[h, s0 + blk]
                    assert np.allclose(y, x[h, r0:r1], rtol=0.07, atol=float(desc[h, s0 + blk]) * 2.0 ** -9)


def test_rotated_block_maxima_match_an_explicit_hadamard():
    # independent rotation: scipy's Sylvester matrix in float64
    rng = np.random.default_rng(4)
    H, D, T, sb = 1, 128, 777, 64
    cu = np.array([0, 64, 65, 400, 777])
    x = _docs_with_spikes(rng, H, cu, D)
    out = varlen.quantize_qkv_varlen(x, x, x, cu, sb, True, 99)
    hm = scipy.linalg.hadamard(D).astype(np.float64)
    y = (x.astype(np.float64) * sign_vector(99, D)) @ hm
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        s0 = varlen.first_slot(cu, d, sb)
        for blk, r0 in enumerate(range(a, b, sb)):
            amax = np.abs(y[0, r0:min(b, r0 + sb)]).max()
            assert abs(out[3][0, s0 + blk] * 448.0 / amax - 1) < 1e-5     # q (rotated)
            vmax = np.abs(x[0, r0:min(b, r0 + sb)]).max()
            # v (never rotated; power-of-two scale): 224 < vmax / descale <= 448
            assert 224.0 < vmax / out[5][0, s0 + blk] <= 448.0


def _masked_attention(q, k, v, cu, causal, scale):
    """softmax over the whole packed sequence with a block-diagonal (and causal) mask."""
    T = q.shape[1]
    doc = np.zeros(T, dtype=np.int64)
    for d in range(len(cu) - 1):
        doc[int(cu[d]):int(cu[d + 1])] = d
    vis = doc[:, None] == doc[None, :]
    if causal:
        vis &= np.arange(T)[None, :] <= np.arange(T)[:, None]
    o = np.empty(q.shape)
    lse = np.empty(q.shape[:2])
    for h in range(q.shape[0]):
        s = (q[h].astype(np.float64) @ k[h].astype(np.float64).T) * scale
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        w = np.exp(s - m[:, None])
        o[h] = (w @ v[h].astype(np.float64)) / w.sum(axis=1)[:, None]
        lse[h] = m + np.log(w.sum(axis=1))
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_reference_is_block_diagonal_attention(causal):
    rng = np.random.default_rng(5)
    H, D, T = 2, 32, 600
    cu = np.array([0, 1, 130, 130, 457, 600])
    q, k, v = (rng.standard_normal((H, T, D)).astype(np.float32) for _ in range(3))
    o, lse = varlen.reference_attention_varlen(q, k, v, cu, causal)
    ob, lb = _masked_attention(q, k, v, cu, causal, 1 / math.sqrt(D))
    assert np.allclose(o, ob, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, lb, rtol=1e-12, atol=1e-12)
    rows = np.array([0, 1, 129, 130, 131, 456, 457, 599])
    o2, l2 = varlen.reference_attention_varlen(q, k, v, cu, causal, rows=rows)
    # (the same values; BLAS may block a shorter product differently)
    assert np.allclose(o2, o[:, rows], rtol=1e-13, atol=1e-13) and np.allclose(l2, lse[:, rows], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sb", [64, 128])
def test_attention_reads_each_documents_slots(causal, sb):
    # arbitrary descales (NaN in the unused slots): the loop without P rounding
    # must equal masked attention of values dequantised by a per-token lookup
    rng = np.random.default_rng(6 + sb)
    H, D, T = 2, 64, 700
    cu = np.array([0, 70, 70, 330, 331, 700])
    ndoc = len(cu) - 1
    codes = [e4m3.encode(rng.standard_normal((H, T, D)) * 30) for _ in range(3)]
    ns = varlen.num_slots(T, ndoc, sb)
    desc = [rng.uniform(0.002, 0.02, (H, ns)) for _ in range(3)]
    used = np.zeros(ns, dtype=bool)
    deq = []
    for i in range(3):
        x = e4m3.decode(codes[i]).copy()
        for t in range(T):
            d = int(np.searchsorted(cu, t, side="right") - 1)
            slot = int(cu[d]) // sb + d + (t - int(cu[d])) // sb
            used[slot] = True
            x[:, t] *= desc[i][:, slot][:, None]
        deq.append(x)
    for i in range(3):
        desc[i][:, ~used] = np.nan
    o, lse = varlen.emulated_fp8_attention_varlen(*codes, *desc, cu, sb, True, causal, quantize_p=False,
                                                  bf16_output=False)
    ob, lb = _masked_attention(*deq, cu, causal, 1 / (math.sqrt(D) * D))
    assert np.allclose(o, ob, rtol=1e-9, atol=1e-9)
    assert np.allclose(lse, lb, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("causal", [False, True])
def test_no_leakage_between_documents(causal):
    rng = np.random.default_rng(8)
    H, D, T = 2, 64, 520
    cu = np.array([0, 200, 330, 520])
    q, k, v = (rng.standard_normal((H, T, D)).astype(np.float32) for _ in range(3))
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for t in (q2, k2, v2):
        t[:, 200:330] = rng.standard_normal((H, 130, D)).astype(np.float32) * 100
    kw = dict(scale_block=128, hadamard=True, seed=3)
    a = varlen.quantize_qkv_varlen(q, k, v, cu, **kw)
    b = varlen.quantize_qkv_varlen(q2, k2, v2, cu, **kw)
    keep = np.r_[0:200, 330:520]
    for i in range(3):
        assert np.array_equal(a[i][:, keep], b[i][:, keep])
    s1 = varlen.first_slot(cu, 1, 128)
    other = [s for s in range(a[3].shape[1]) if s not in (s1, s1 + 1)]
    for i in range(3, 6):
        assert np.array_equal(a[i][:, other], b[i][:, other], equal_nan=True)
        assert not np.array_equal(a[i][:, s1], b[i][:, s1])
    oa, la = varlen.emulated_fp8_attention_varlen(*a, cu, 128, True, causal)
    ob, lb = varlen.emulated_fp8_attention_varlen(*b, cu, 128, True, causal)
    assert np.array_equal(oa[:, keep], ob[:, keep]) and np.array_equal(la[:, keep], lb[:, keep])


def test_one_document_is_the_dense_path():
    rng = np.random.default_rng(9)
    H, D, T = 2, 64, 333
    q, k, v = (rng.standard_normal((H, T, D)).astype(np.float32) for _ in range(3))
    from oracle.quantize import quantize_qkv
    a = varlen.quantize_qkv_varlen(q, k, v, [0, T], 64, True, 5, pow2=True)
    b = quantize_qkv(q, k, v, 64, True, 5, pow2=True)
    nb = -(-T // 64)
    for i in range(3):
        assert np.array_equal(a[i], b[i])
        assert np.array_equal(a[3 + i][:, :nb], b[3 + i]) and np.all(np.isnan(a[3 + i][:, nb:]))
    oa, la = varlen.emulated_fp8_attention_varlen(*a[:3], *(x[:, :nb] for x in a[3:]), [0, T], 64, True, True)
    ob, lb = attention.emulated_fp8_attention_tiled(*b, 64, True, True)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_cu_seqlens_is_checked():
    x = np.zeros((1, 10, 64), dtype=np.float32)
    for cu in ([0, 5], [1, 10], [0, 6, 5, 10], [0, 11]):
        with pytest.raises(ValueError):
            varlen.quantize_qkv_varlen(x, x, x, cu, 64, False, 0)


@pytest.mark.parametrize("causal", [False, True])
def test_work_items(causal):
    rng = np.random.default_rng(10)
    for trial in range(50):
        T = int(rng.integers(1, 5000))
        cu = _random_cu(rng, T, int(rng.integers(1, 12)))
        lf = varlen.work_items(cu, causal)
        nat = varlen.work_items(cu, causal, order="natural")
        # every (document, query tile) exactly once, in both orders
        brute = []
        for d in range(len(cu) - 1):
            L = int(cu[d + 1] - cu[d])
            r = 0
            while r * 128 < L:
                last_q = min(L, 128 * (r + 1)) - 1          # the tile's last query
                keys = last_q + 1 if causal else L           # keys it sees
                brute.append((d, r, -(-keys // 128)))
                r += 1
        assert sorted(lf) == sorted(brute) and nat == brute
        # longest first: documents by non-increasing tile count, each one's
        # tiles together and descending (so the costliest causal tile first)
        docs = [d for i, (d, _, _) in enumerate(lf) if i == 0 or lf[i - 1][0] != d]
        assert len(docs) == len(set(docs))
        nts = [sum(1 for it in brute if it[0] == d) for d in docs]
        assert all(x >= y for x, y in zip(nts, nts[1:]))
        for d in docs:
            rs = [r for dd, r, _ in lf if dd == d]
            assert rs == sorted(rs, reverse=True)
        if causal and lf:
            assert lf[0][2] == max(c for _, _, c in brute)
