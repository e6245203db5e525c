"""Packed variable-length documents (oracle; test infrastructure only).

[P3] "FLAMIA ..." (paperlayer.ai summary of arXiv 2611.03344v1), Abstract and
4.1 Performance on Packed Documents: documents of different lengths are packed
one after another, with no padding and no repacking; scales are local to a
document (document-local scaling); the scheduler orders the work so that the
longest items start first (4.3 Ablation Study: removing longest-first order
costs 10-65% of the causal forward time).  F. System Integration: the work
lists live on the GPU.

The pages leave the layout and the block rule open.  Readings taken here:
  * layout [H][T][D]: heads outermost; in every head the T packed tokens in
    document order.  Document d holds tokens cu[d] .. cu[d+1]-1, where cu has
    ndoc + 1 non-decreasing entries from 0 to T (empty documents allowed);
  * a scale block never crosses a document boundary: the blocks of a document
    are its tokens in groups of ``scale_block`` counted from its first token,
    the last one possibly short, i.e. the dense rule of ``quantize`` applied
    to each document as a sequence of its own;
  * the descale of block b of document d sits at index cu[d] // scale_block +
    d + b of a head's row of T // scale_block + ndoc entries.  This needs no
    prefix sum over documents; the entries it skips are not written;
  * attention, causal or not, runs inside each document; causal: a query sees
    the keys of its own document up to its own position;
  * work item = (document, query tile of 128 queries); its cost is the number
    of key tiles it visits: r + 1 for tile r of a causal document, the
    document's tile count otherwise.  Longest-first is read at the grain of
    documents: documents in non-increasing tile count, each one's items
    together, its tiles from the last (the costliest under a causal mask) to
    the first; the order among documents of equal tile count is free.  The
    natural order (the ablation's baseline) is document-major, tiles
    ascending.
"""

import math

import numpy as np

from .attention import emulated_fp8_attention_bars, emulated_fp8_attention_tiled, reference_attention
from .quantize import quantize_qkv

QUERY_TILE = 128


def check_cu(cu, T):
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or len(cu) < 2 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing from 0 to T")
    return cu


def num_slots(T, ndoc, scale_block):
    """Descale entries per head."""
    return T // scale_block + ndoc


def first_slot(cu, d, scale_block):
    """Index of the first descale of document d in a head's row."""
    return int(cu[d]) // scale_block + d


def quantize_qkv_varlen(q, k, v, cu, scale_block, hadamard, seed, pow2=False):
    """Rotate + document-local block scale + e4m3 of packed Q, K, V [H, T, D].

    Returns (q8, k8, v8 [H, T, D] uint8, q/k/v descale [H, num_slots] float32);
    descale entries that belong to no block are NaN.
    """
    H, T, D = np.shape(q)
    cu = check_cu(cu, T)
    ndoc = len(cu) - 1
    codes = [np.zeros((H, T, D), dtype=np.uint8) for _ in range(3)]
    desc = [np.full((H, num_slots(T, ndoc, scale_block)), np.nan, dtype=np.float32) for _ in range(3)]
    for d in range(ndoc):
        a, b = int(cu[d]), int(cu[d + 1])
        if a == b:
            continue
        out = quantize_qkv(q[:, a:b], k[:, a:b], v[:, a:b], scale_block, hadamard, seed, pow2)
        s0 = first_slot(cu, d, scale_block)
        for i in range(3):
            codes[i][:, a:b] = out[i]
            desc[i][:, s0:s0 + out[3 + i].shape[-1]] = out[3 + i]
    return (*codes, *desc)


def _doc_rows(cu, rows, T):
    """Group packed token indices by document: {d: (local rows, positions in rows)}."""
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    doc = np.searchsorted(cu, rows, side="right") - 1
    out = {}
    for d in np.unique(doc):
        pos = np.nonzero(doc == d)[0]
        out[int(d)] = (rows[pos] - cu[d], pos)
    return rows, out


def reference_attention_varlen(q, k, v, cu, causal, rows=None):
    """Exact float64 attention of each document of packed [H, T, D] inputs.

    ``rows``: packed token indices to evaluate (all by default).  Returns
    (O [H, R, D], LSE [H, R]).
    """
    H, T, D = np.shape(q)
    cu = check_cu(cu, T)
    rows, groups = _doc_rows(cu, rows, T)
    o = np.empty((H, len(rows), D))
    lse = np.empty((H, len(rows)))
    for d, (loc, pos) in groups.items():
        a, b = int(cu[d]), int(cu[d + 1])
        od, ld = reference_attention(q[:, a:b], k[:, a:b], v[:, a:b], causal, rows=loc)
        o[:, pos] = od
        lse[:, pos] = ld
    return o, lse


def emulated_fp8_attention_varlen(q8, k8, v8, q_descale, k_descale, v_descale, cu, scale_block, hadamard,
                                  causal, rows=None, **kw):
    """E2 (``attention.emulated_fp8_attention_tiled``) of each packed document.

    Each document is a sequence of its own: its codes, and the descales of its
    blocks read from its slots.  Keyword options (tau, quantize_p, bf16_output,
    block_c, exp2, lift) pass through.  Returns (O [H, R, D], LSE [H, R]).
    """
    H, T, D = np.shape(q8)
    cu = check_cu(cu, T)
    rows, groups = _doc_rows(cu, rows, T)
    o = np.empty((H, len(rows), D))
    lse = np.empty((H, len(rows)))
    for d, (loc, pos) in groups.items():
        a, b = int(cu[d]), int(cu[d + 1])
        s0 = first_slot(cu, d, scale_block)
        nb = -(-(b - a) // scale_block)
        sl = slice(s0, s0 + nb)
        res = emulated_fp8_attention_tiled(q8[:, a:b], k8[:, a:b], v8[:, a:b], q_descale[:, sl],
                                           k_descale[:, sl], v_descale[:, sl], scale_block, hadamard, causal,
                                           rows=loc, **kw)
        o[:, pos] = res[0]
        lse[:, pos] = res[1]
    return o, lse


def emulated_fp8_attention_varlen_bars(q8, k8, v8, q_descale, k_descale, v_descale, cu, scale_block, hadamard,
                                       causal, rows=None, exp2="exact"):
    """E1 of each packed document with the FP8 error bars of
    ``attention.emulated_fp8_attention_bars``: each document is a sequence of
    its own (its codes and the descales of its blocks, read from its slots).
    Returns the same dict, O and the bars [H, R, D], LSE and its bar [H, R]."""
    H, T, D = np.shape(q8)
    cu = check_cu(cu, T)
    rows, groups = _doc_rows(cu, rows, T)
    out = {key: np.empty((H, len(rows), D)) for key in ("o", "pbar", "sigma", "acc_bar")}
    out.update({key: np.empty((H, len(rows))) for key in ("lse", "lse_bar")})
    for d, (loc, pos) in groups.items():
        a, b = int(cu[d]), int(cu[d + 1])
        s0 = first_slot(cu, d, scale_block)
        sl = slice(s0, s0 + -(-(b - a) // scale_block))
        res = emulated_fp8_attention_bars(q8[:, a:b], k8[:, a:b], v8[:, a:b], q_descale[:, sl], k_descale[:, sl],
                                          v_descale[:, sl], scale_block, hadamard, causal, rows=loc, exp2=exp2)
        for key in out:
            out[key][:, pos] = res[key]
    return out


def work_items(cu, causal, order="longest_first"):
    """The (document, query tile) items of one head and their costs, in ``order``.

    Returns a list of (doc, tile, cost).  "longest_first": documents in
    non-increasing tile count (ties by document index here; any order of
    ties is valid), each document's tiles together and descending;
    "natural": document-major, tiles ascending.
    """
    cu = np.asarray(cu, dtype=np.int64)
    nts = [math.ceil(int(cu[d + 1] - cu[d]) / QUERY_TILE) for d in range(len(cu) - 1)]
    if order == "longest_first":
        docs = sorted(range(len(nts)), key=lambda d: (-nts[d], d))
        tiles = lambda nt: range(nt - 1, -1, -1)
    elif order == "natural":
        docs = range(len(nts))
        tiles = lambda nt: range(nt)
    else:
        raise ValueError("order must be 'longest_first' or 'natural'")
    return [(d, r, r + 1 if causal else nts[d]) for d in docs for r in tiles(nts[d])]
