"""The balanced decode schedule's integer rules, restated on the CPU (host
logic; the GPU tests run the kernels themselves).

The 64-key tiles of every (sequence, K/V head) form one flat order
(sequence-major, then head, then tile) of T tiles; W waves (W <= T) take the
shares [floor(w T / W), floor((w + 1) T / W)).  A share spanning several
(sequence, head) segments makes one piece per segment, and the piece of wave
w in segment s writes its partial to slot w + s.  The merge of segment s
reads the slots w + s for the waves from the one holding the segment's first
tile to the one holding its last, ceil((x + 1) W / T) - 1 for tile x.

Checked on random batches (lengths 0..Ncap, empty sequences, more waves than
tiles): every key of every segment is covered exactly once, slots are
distinct and inside the W + B * Hkv the workspace holds, and the merge reads
exactly the slots that were written (none left unwritten between them).
"""

import numpy as np
import pytest

import fp8_attention_forward_amd as fa

TILE = 64


def _waves(B, Hkv, Ncap):
    tmax = B * Hkv * (-(-Ncap // TILE))
    w = min(2048, tmax)
    return -(-w // 4) * 4


def _pieces(L, Hkv, W):
    nt = -(-L // TILE)
    seg_tiles = np.repeat(nt, Hkv)                    # segment s = b * Hkv + hk
    start = np.concatenate([[0], np.cumsum(seg_tiles)])
    T = int(start[-1])
    W = min(W, T)
    pieces = []
    for w in range(W):
        x, x1 = T * w // W, T * (w + 1) // W
        assert x1 > x
        while x < x1:
            s = int(np.searchsorted(start, x, side="right")) - 1
            tile = x - int(start[s])
            n = min(x1 - x, int(seg_tiles[s]) - tile)
            b, hk = divmod(s, Hkv)
            k0, k1 = tile * TILE, min(int(L[b]), (tile + n) * TILE)
            pieces.append((w, s, k0, k1))
            x += n
    return pieces, T, W, start, seg_tiles


def _merge_slots(s, T, W, start, seg_tiles):
    if seg_tiles[s] == 0:
        return []
    wave_of = lambda x: -(-((x + 1) * W) // T) - 1
    x0 = int(start[s])
    wf, wl = wave_of(x0), wave_of(x0 + int(seg_tiles[s]) - 1)
    return list(range(wf + s, wl + s + 1))


@pytest.mark.parametrize("seed", range(40))
def test_shares_cover_each_key_once_and_the_merge_reads_what_was_written(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 5, 16, 63, 64, 65, 200, 512]))
    Hkv = int(rng.integers(1, 9))
    Ncap = int(rng.choice([1, 63, 64, 65, 300, 2048]))
    L = rng.integers(0, Ncap + 1, size=B)
    if rng.random() < 0.3:
        L[rng.random(B) < 0.5] = 0
    W = _waves(B, Hkv, Ncap)
    pieces, T, Weff, start, seg_tiles = _pieces(L, Hkv, W)
    slots = [w + s for w, s, _, _ in pieces]
    assert len(set(slots)) == len(slots)
    assert all(0 <= x < W + B * Hkv for x in slots)
    covered = {}
    for w, s, k0, k1 in pieces:
        assert 0 <= k0 < k1
        covered[s] = covered.get(s, 0) + (k1 - k0)
        assert covered[s] <= L[s // Hkv]
    for s in range(B * Hkv):
        assert covered.get(s, 0) == L[s // Hkv]
        written = sorted(w + s2 for w, s2, _, _ in pieces if s2 == s)
        assert written == _merge_slots(s, T, Weff, start, seg_tiles)


def test_workspace_holds_every_slot():
    # the library's workspace size is the slot count of this rule times the
    # per-slot bytes (MQ rows of D + 2 floats)
    for B, Hq, Hkv, Sq, Ncap, D in ((16, 32, 8, 1, 32768, 128), (3, 8, 2, 2, 3000, 128), (1, 1, 1, 1, 64, 64)):
        mq = Hq // Hkv * Sq
        assert fa.attn_fp8_decode_workspace_bytes(B, Hq, Hkv, Sq, Ncap, D) == \
            4 * (_waves(B, Hkv, Ncap) + B * Hkv) * mq * (D + 2)
