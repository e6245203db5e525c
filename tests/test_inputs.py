"""The seeded input kinds do what their tests rely on (CPU)."""

import math

import numpy as np

import workloads
from oracle import e4m3
from oracle import quantize as oq


def test_ramp_scores_rise_on_consecutive_key_tiles():
    # The lazy reference moves when a 64-key tile's largest scaled score (log2
    # units) exceeds the reference by more than 8.8, and then sits 2 below that
    # maximum; so a tile maximum that rises by more than 6.8 over the previous
    # one moves the reference again.  The ramp kind must give such runs for
    # every query on the quantised inputs the kernel sees.
    for (N, D, sb, had) in ((700, 128, 128, True), (640, 64, 64, False)):
        q, k, v = workloads.generate("ramp", 1, 2, N, D, 200 + N)
        q8, k8, _, qd, kd, _ = oq.quantize_qkv(q, k, v, sb, had, 0x5EED)
        for h in range(2):
            qq = e4m3.decode(q8[0, h]).astype(np.float64) * np.repeat(qd[0, h], sb)[:N, None]
            kk = e4m3.decode(k8[0, h]).astype(np.float64) * np.repeat(kd[0, h], sb)[:N, None]
            t = qq @ kk.T * (math.log2(math.e) / math.sqrt(D) / (D if had else 1))
            nt = -(-N // 64)
            tmax = np.stack([t[:, 64 * j:64 * j + 64].max(axis=1) for j in range(nt)], axis=1)
            rises = np.diff(tmax, axis=1) > 6.8
            assert rises.all(), (N, D, h, rises.mean())
