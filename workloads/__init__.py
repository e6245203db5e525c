"""Seeded synthetic inputs for the FP8 attention forward pass.

Shared by the oracle-based tests and by the GPU path's tests and benchmark.
This module holds no arithmetic of the method: it only draws Q, K, V (float32,
layout [B][H][N][D]) from numpy's PCG64 generator.

The pages measure on captured activations of two named open-weights models on
a fixed 8k-token text plus FlashAttention-3's synthetic outlier test ([P1]
"FP8 attention that keeps FlashAttention-3 throughput at BF16-level accuracy",
"How it gets verified"; [P2] "Fused attention kernel", 8-bit forward pass).
The captured activations, weights and text are not available, so every
workload here is synthetic and stands in for them:
  * ``outlier``: iid N(0,1) with 0.1% of entries replaced by N(0, 10^2)
    ([P2] 8-bit forward pass: 0.1% outlier entries; the outlier distribution is
    not stated on the pages, N(0, 10^2) is the reading taken here);
  * ``channel``: LLM-like channel outliers: Q and K are N(0,1) with 4 channels
    per head (the same for Q and K, every batch and token) set to 30 z + 5;
    V is Student-t with 4 degrees of freedom;
  * ``iid``: iid N(0,1).

Draw order (fixed): Q, K, V base values; then per tensor the outlier mask and
outlier values (``outlier``), or the per-head channel ids (``channel``).
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, asdict

import numpy as np

SIGN_SEED = 0x5EED     # seed of the random sign diagonal in every configuration


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    causal: bool
    scale_block: int
    hadamard: bool
    kind: str          # "iid" | "outlier" | "channel"
    data_seed: int
    sign_seed: int = SIGN_SEED

    def as_dict(self):
        return asdict(self)

    def flops(self):
        """Algorithmic FLOPs: 4 d per visible (query, key) pair."""
        pairs = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return 4 * self.D * self.B * self.H * pairs


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 64, False, 64, True, "iid", 0),
    "outlier": Workload("outlier", 2, 32, 8192, 128, False, 128, True, "outlier", 1),
    "outlier_causal": Workload("outlier_causal", 2, 32, 8192, 128, True, 128, True, "outlier", 1),
    "ablation": Workload("ablation", 4, 16, 8448, 128, False, 128, True, "iid", 3),
    "ablation_tail": Workload("ablation_tail", 4, 16, 8400, 128, False, 128, True, "iid", 3),
    "channel": Workload("channel", 2, 32, 8192, 128, True, 128, True, "channel", 4),
    "channel_norot": Workload("channel_norot", 2, 32, 8192, 128, True, 128, False, "channel", 4),
}


def generate(kind, B, H, N, D, seed):
    """(q, k, v) float32 arrays of shape [B, H, N, D]."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, D)
    q = rng.standard_normal(size=shape, dtype=np.float32)
    k = rng.standard_normal(size=shape, dtype=np.float32)
    if kind == "channel":
        v = rng.standard_t(4, size=shape).astype(np.float32)
    else:
        v = rng.standard_normal(size=shape, dtype=np.float32)
    if kind == "outlier":
        for t in (q, k, v):
            mask = rng.random(size=shape, dtype=np.float32) < 0.001
            cnt = int(mask.sum())
            t[mask] = (10.0 * rng.standard_normal(size=cnt, dtype=np.float32)).astype(np.float32)
    elif kind == "channel":
        for h in range(H):
            ch = rng.choice(D, size=4, replace=False)
            for t in (q, k):
                t[:, h, :, ch] = np.float32(30.0) * t[:, h, :, ch] + np.float32(5.0)
    elif kind == "ramp":
        # Q and K share one unit direction u per head; K's component along u
        # grows by 0.25 per token, so every query's scores rise along the keys
        # (by about 16 log2 units per 64-key tile at D = 128 with Q's 10 u):
        # the running maximum climbs on every key tile
        u = rng.standard_normal(size=(B, H, 1, D)).astype(np.float32)
        u /= np.linalg.norm(u, axis=-1, keepdims=True).astype(np.float32)
        q += np.float32(10.0) * u
        k += (np.float32(0.25) * np.arange(N, dtype=np.float32))[None, None, :, None] * u
    elif kind != "iid":
        raise ValueError(f"unknown workload kind {kind!r}")
    return q, k, v


def generate_workload(w: Workload):
    return generate(w.kind, w.B, w.H, w.N, w.D, w.data_seed)


# ---------------------------------------------------------------------------
# Packed variable-length documents ([P3] FLAMIA, 4.1 Performance on Packed
# Documents: 16 query heads, d = 128, up to T = 131072 packed tokens; its
# workloads include equal-length and skewed length mixes, 4.3 Ablation Study).
# The pages do not list the document lengths, so three seeded mixes stand in:
#   * ``equal:L``: T / L documents of L tokens;
#   * ``skewed:LO:HI``: lengths drawn log-uniformly from [LO, HI] until T is
#     filled (the last document takes what is left);
#   * ``long:F``: one document of F * T tokens first, then lengths drawn
#     log-uniformly from [64, 2048] for the rest.
# Layout [H][T][D] (heads outermost, packed tokens in document order);
# cu_seqlens = [0, l_0, l_0 + l_1, ..., T] as int32.


@dataclass(frozen=True)
class PackedWorkload:
    name: str
    H: int
    T: int
    D: int
    causal: bool
    scale_block: int
    hadamard: bool
    kind: str          # value distribution, as for Workload
    data_seed: int
    mix: str           # length mix, see above
    len_seed: int = 0
    sign_seed: int = SIGN_SEED

    def as_dict(self):
        return asdict(self)

    def cu_seqlens(self):
        return cu_seqlens(doc_lengths(self.mix, self.T, self.len_seed))

    def flops(self):
        """Algorithmic FLOPs: 4 d per visible (query, key) pair, summed over documents."""
        lens = np.diff(self.cu_seqlens()).astype(np.int64)
        pairs = lens * (lens + 1) // 2 if self.causal else lens * lens
        return int(4 * self.D * self.H * pairs.sum())


def doc_lengths(mix, T, seed):
    """Document lengths (int64 array summing to T) of a length mix."""
    kind, _, arg = mix.partition(":")
    rng = np.random.default_rng(seed)
    if kind == "equal":
        L = int(arg)
        lens = [L] * (T // L) + ([T % L] if T % L else [])
    elif kind in ("skewed", "long"):
        lens = []
        if kind == "long":
            first = int(float(arg) * T)
            lens.append(first)
            lo, hi = 64, 2048
        else:
            lo, hi = (int(x) for x in arg.split(":"))
        left = T - sum(lens)
        while left > 0:
            n = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
            n = min(max(n, 1), left)
            lens.append(n)
            left -= n
    else:
        raise ValueError(f"unknown length mix {mix!r}")
    return np.asarray(lens, dtype=np.int64)


def cu_seqlens(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


PACKED_WORKLOADS = {
    "packed_skewed_causal": PackedWorkload("packed_skewed_causal", 16, 131072, 128, True, 128, True, "iid", 5,
                                           "skewed:256:32768", 1),
    "packed_equal_causal": PackedWorkload("packed_equal_causal", 16, 131072, 128, True, 128, True, "iid", 5,
                                          "equal:4096"),
    "packed_long_causal": PackedWorkload("packed_long_causal", 16, 131072, 128, True, 128, True, "iid", 5,
                                         "long:0.5", 2),
    "packed_skewed": PackedWorkload("packed_skewed", 16, 131072, 128, False, 128, True, "iid", 5,
                                    "skewed:256:32768", 1),
}


def generate_packed(kind, H, T, D, seed):
    """(q, k, v) float32 arrays of shape [H, T, D].

    Every (tensor, head) slice has its own PCG64 stream, child i = 3 * h + t
    (t = 0, 1, 2 for Q, K, V) of SeedSequence(seed): its N(0, 1) base values,
    then for ``outlier`` its 0.1% mask and N(0, 10^2) outlier values.  The
    slices are independent, so they are drawn on several threads.
    """
    if kind not in ("iid", "outlier"):
        raise ValueError(f"packed inputs support the iid and outlier kinds, not {kind!r}")
    out = np.empty((3, H, T, D), dtype=np.float32)
    children = np.random.SeedSequence(seed).spawn(3 * H)

    def draw(i):
        h, t = divmod(i, 3)
        rng = np.random.default_rng(children[i])
        x = out[t, h]
        rng.standard_normal(size=(T, D), dtype=np.float32, out=x)
        if kind == "outlier":
            mask = rng.random(size=(T, D), dtype=np.float32) < 0.001
            x[mask] = (10.0 * rng.standard_normal(size=int(mask.sum()), dtype=np.float32)).astype(np.float32)

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(draw, range(3 * H)))
    return out[0], out[1], out[2]


def generate_packed_workload(w: PackedWorkload):
    return generate_packed(w.kind, w.H, w.T, w.D, w.data_seed)


# ---------------------------------------------------------------------------
# Decode against an FP8 K/V cache ([P1] Realistic applications: FP8 K and V
# relieve KV-cache bandwidth).  The pages give no decode workload; the stand-in
# is a batch of sequences of mixed lengths with grouped query heads (G query
# heads per K/V head), one new token each, head dimension 128.


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Ncap: int
    D: int
    causal: bool
    scale_block: int
    hadamard: bool
    kind: str
    data_seed: int
    len_lo: int        # sequence lengths drawn uniformly from [len_lo, Ncap]
    len_seed: int = 0
    sign_seed: int = SIGN_SEED

    def as_dict(self):
        return asdict(self)

    def seqlens(self):
        rng = np.random.default_rng(self.len_seed)
        return rng.integers(self.len_lo, self.Ncap + 1, size=self.B).astype(np.int32)

    def kv_bytes(self):
        """Bytes of K and V codes a decode step reads: 2 D per cached token and K/V head."""
        return int(2 * self.D * self.Hkv * self.seqlens().astype(np.int64).sum())

    def flops(self):
        """4 d per visible (query, key) pair."""
        L = self.seqlens().astype(np.int64)
        pairs = (self.Sq * L - self.Sq * (self.Sq - 1) // 2) if self.causal else self.Sq * L
        return int(4 * self.D * self.Hq * pairs.sum())


DECODE_WORKLOADS = {
    "decode_gqa": DecodeWorkload("decode_gqa", 16, 32, 8, 1, 32768, 128, True, 128, True, "iid", 7, 1024, 3),
    "decode_gqa_spec": DecodeWorkload("decode_gqa_spec", 16, 32, 8, 4, 32768, 128, True, 128, True, "iid", 7, 1024, 3),
}


def generate_decode(kind, B, Hq, Hkv, Sq, Ncap, D, seed):
    """(q [B, Hq, Sq, D], k [B, Hkv, Ncap, D], v [B, Hkv, Ncap, D]) float32.

    Each (tensor, batch, head) slice has its own PCG64 stream, children of
    SeedSequence(seed) in the order q slices, k slices, v slices (batch-major),
    drawn as in ``generate_packed`` on several threads.
    """
    if kind not in ("iid", "outlier"):
        raise ValueError(f"decode inputs support the iid and outlier kinds, not {kind!r}")
    q = np.empty((B, Hq, Sq, D), dtype=np.float32)
    k = np.empty((B, Hkv, Ncap, D), dtype=np.float32)
    v = np.empty((B, Hkv, Ncap, D), dtype=np.float32)
    slices = [(q, b, h) for b in range(B) for h in range(Hq)] + \
        [(t, b, h) for t in (k, v) for b in range(B) for h in range(Hkv)]
    children = np.random.SeedSequence(seed).spawn(len(slices))

    def draw(j):
        t, b, h = slices[j]
        rng = np.random.default_rng(children[j])
        x = t[b, h]
        rng.standard_normal(size=x.shape, dtype=np.float32, out=x)
        if kind == "outlier":
            mask = rng.random(size=x.shape, dtype=np.float32) < 0.001
            x[mask] = (10.0 * rng.standard_normal(size=int(mask.sum()), dtype=np.float32)).astype(np.float32)

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(draw, range(len(slices))))
    return q, k, v


def generate_decode_workload(w: DecodeWorkload):
    return generate_decode(w.kind, w.B, w.Hq, w.Hkv, w.Sq, w.Ncap, w.D, w.data_seed)
