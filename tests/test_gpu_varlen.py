"""GPU parity of the packed variable-length document path against the oracle.

* quantize_qkv_fp8_varlen: codes and the descales of every block bit-exact
  against oracle.varlen (document-local blocks, slot layout).
* attn_fp8_fwd_varlen: O and LSE against E1 of every document (the exact
  attention of its quantised inputs), with the dense path's bars
  (tests.gpu_common.check_fp8_vs_e1); both work orders give the same bits.
* One document equals the dense path bit for bit, and every document equals
  the dense path run on that document alone.
* The work list in the workspace: every (document, query tile) once; longest
  first = documents by non-increasing length, each one's tiles together and
  descending; or document-major (natural order).
* cu_seqlens that break the rule: status 1, nothing written.
"""

import numpy as np
import pytest
import torch

import fp8_attention_forward_amd as fa
import workloads
from oracle import varlen as ov
from tests.gpu_common import check_fp8_vs_e1, dev, host, rms, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _lens_cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _random_cu(n, lo, hi, seed):
    rng = np.random.default_rng(seed)
    return _lens_cu(rng.integers(lo, hi + 1, size=n))


CASES = [
    # H, D, scale_block, hadamard, causal, cu_seqlens, kind
    (2, 64, 64, True, False, [0, 300, 300, 428, 1000], "iid"),
    (2, 128, 128, True, True, [0, 1, 2, 130, 259, 900], "outlier"),
    (1, 128, 64, False, True, [0, 64, 128, 192, 1000], "iid"),
    (3, 64, 128, True, True, _random_cu(20, 1, 300, 1), "iid"),
    (2, 128, 128, True, False, [0, 700], "outlier"),
    (2, 128, 128, True, True, _random_cu(150, 1, 10, 2), "iid"),
    (1, 128, 128, True, False, [0, 0, 0, 517, 517, 1300, 1300], "outlier"),
    (2, 64, 64, False, False, _random_cu(7, 100, 700, 3), "outlier"),
]
IDS = ["H{}D{}sb{}had{}c{}-nd{}".format(c[0], c[1], c[2], int(c[3]), int(c[4]), len(c[5]) - 1) for c in CASES]


def _inputs(case, seed_off=0):
    H, D, sb, had, causal, cu, kind = case
    cu = np.asarray(cu, dtype=np.int32)
    T = int(cu[-1])
    q, k, v = workloads.generate_packed(kind, H, T, D, 40 + T + seed_off)
    return q, k, v, cu


def _used_slots(cu, T, sb):
    used = np.zeros(ov.num_slots(T, len(cu) - 1, sb), dtype=bool)
    for d in range(len(cu) - 1):
        nb = -(-(int(cu[d + 1]) - int(cu[d])) // sb)
        s0 = ov.first_slot(cu, d, sb)
        used[s0:s0 + nb] = True
    return used


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_quantize_varlen_bit_exact(case, pow2):
    H, D, sb, had, causal, _, kind = case
    q, k, v, cu = _inputs(case)
    T = int(cu[-1])
    print(f"\n[quantize varlen] {case[:5]} ndoc {len(cu) - 1} T {T} pow2 {pow2}", flush=True)
    out = fa.quantize_qkv_fp8_varlen(dev(q), dev(k), dev(v), dev(cu), scale_block=sb, hadamard=had, seed=0x5EED,
                                     mx=pow2)
    torch.cuda.synchronize()
    ref = ov.quantize_qkv_varlen(q, k, v, cu, sb, had, 0x5EED, pow2=pow2)
    used = _used_slots(cu, T, sb)
    for g, r, nm in zip((host(t) for t in out), ref, ("q8", "k8", "v8", "qd", "kd", "vd")):
        if r.dtype == np.uint8:
            assert np.array_equal(g, r), f"{nm}: {np.count_nonzero(g != r)} codes differ"
        else:
            assert np.all(np.isnan(r[:, ~used]))
            assert np.array_equal(g[:, used].view(np.uint32), r[:, used].view(np.uint32)), f"{nm}: descales differ"


def _gpu_varlen(case, q, k, v, cu, order="longest_first", exp2="exact", mx=False, ws=None):
    H, D, sb, had, causal, _, _ = case
    cu_d = dev(cu)
    qq = fa.quantize_qkv_fp8_varlen(dev(q), dev(k), dev(v), cu_d, scale_block=sb, hadamard=had, seed=0x5EED, mx=mx)
    o, lse = fa.attn_fp8_fwd_varlen(*qq, cu_d, scale_block=sb, hadamard=had, causal=causal, exp2=exp2, mx=mx,
                                    order=order, workspace=ws)
    torch.cuda.synchronize()
    return qq, host(o), host(lse)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_attn_varlen_matches_e1(case):
    H, D, sb, had, causal, _, kind = case
    q, k, v, cu = _inputs(case)
    print(f"\n[attn varlen] {case[:5]} ndoc {len(cu) - 1} T {int(cu[-1])}", flush=True)
    _, o, lse = _gpu_varlen(case, q, k, v, cu)
    _, o_nat, lse_nat = _gpu_varlen(case, q, k, v, cu, order="natural")
    assert np.array_equal(o, o_nat) and np.array_equal(lse, lse_nat), "the work order changed a result"
    ref = ov.quantize_qkv_varlen(q, k, v, cu, sb, had, 0x5EED)
    check_fp8_vs_e1(o, lse, ov.emulated_fp8_attention_varlen_bars(*ref, cu, sb, had, causal), tag=f"{case[:5]} varlen")
    o2, _ = ov.emulated_fp8_attention_varlen(*ref, cu, sb, had, causal)
    print(f"  diagnostic RMSE vs E2 {rms(o - o2):.3e}", flush=True)


@pytest.mark.parametrize("exp2,mx", [("schraudolph", False), ("exact", True), ("schraudolph", True)])
@pytest.mark.parametrize("case", [CASES[1], CASES[3], CASES[4]], ids=[IDS[1], IDS[3], IDS[4]])
def test_attn_varlen_options_match_e1(case, exp2, mx):
    H, D, sb, had, causal, _, kind = case
    q, k, v, cu = _inputs(case, seed_off=7)
    print(f"\n[attn varlen {exp2} mx={mx}] {case[:5]} ndoc {len(cu) - 1}", flush=True)
    _, o, lse = _gpu_varlen(case, q, k, v, cu, exp2=exp2, mx=mx)
    ref = ov.quantize_qkv_varlen(q, k, v, cu, sb, had, 0x5EED, pow2=mx)
    check_fp8_vs_e1(o, lse, ov.emulated_fp8_attention_varlen_bars(*ref, cu, sb, had, causal, exp2=exp2),
                    tag=f"{case[:5]} {exp2} mx={mx}")


@pytest.mark.parametrize("causal", [False, True])
def test_one_document_is_the_dense_path_bitwise(causal):
    H, T, D, sb = 2, 777, 128, 128
    q, k, v = workloads.generate_packed("outlier", H, T, D, 11)
    cu = np.array([0, T], dtype=np.int32)
    qv = fa.quantize_qkv_fp8_varlen(dev(q), dev(k), dev(v), dev(cu), scale_block=sb, seed=0x5EED)
    qd = fa.quantize_qkv_fp8(dev(q[None]), dev(k[None]), dev(v[None]), scale_block=sb, seed=0x5EED)
    nb = -(-T // sb)
    for a, b in zip(qv[:3], qd[:3]):
        assert torch.equal(a, b[0])
    for a, b in zip(qv[3:], qd[3:]):
        assert torch.equal(a[:, :nb], b[0])
    ov_, lv = fa.attn_fp8_fwd_varlen(*qv, dev(cu), scale_block=sb, causal=causal)
    od, ld = fa.attn_fp8_fwd(*qd, scale_block=sb, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(ov_, od[0]) and torch.equal(lv, ld[0])


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[3], CASES[7]], ids=[IDS[0], IDS[1], IDS[3], IDS[7]])
def test_every_document_is_the_dense_path_bitwise(case):
    # the dense kernel on one document's rows and blocks gives the same bits
    H, D, sb, had, causal, _, _ = case
    q, k, v, cu = _inputs(case, seed_off=3)
    qq, o, lse = _gpu_varlen(case, q, k, v, cu)
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        if a == b:
            continue
        s0 = ov.first_slot(cu, d, sb)
        nb = -(-(b - a) // sb)
        doc = [t[:, a:b].contiguous()[None] for t in qq[:3]] + [t[:, s0:s0 + nb].contiguous()[None] for t in qq[3:]]
        od, ld = fa.attn_fp8_fwd(*doc, scale_block=sb, hadamard=had, causal=causal)
        torch.cuda.synchronize()
        assert np.array_equal(host(od)[0], o[:, a:b]) and np.array_equal(host(ld)[0], lse[:, a:b]), f"document {d}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", ["longest_first", "natural"])
def test_work_list(causal, order):
    rng = np.random.default_rng(5)
    cu = _lens_cu(np.concatenate([rng.integers(0, 1500, 60), [3000]]))   # empty ones, and a long one last
    T = int(cu[-1])
    H, D, sb = 1, 64, 64
    case = (H, D, sb, True, causal, cu, "iid")
    q, k, v = workloads.generate_packed("iid", H, T, D, 6)
    ws = torch.full((fa.attn_fp8_varlen_workspace_bytes(T, len(cu) - 1),), 0xAB, dtype=torch.uint8, device="cuda")
    _gpu_varlen(case, q, k, v, cu, order=order, ws=ws)
    w = ws.cpu().numpy().view(np.int32)
    count, status = int(w[0]), int(w[1])
    items = [tuple(int(x) for x in w[4 + 2 * i: 6 + 2 * i]) for i in range(count)]
    ref = ov.work_items(cu, causal, order=order)
    assert status == 0 and count == len(ref)
    if order == "natural":
        assert items == [(d, r) for d, r, _ in ref]
    else:
        # the same items; documents in non-increasing tile count, each one's
        # tiles together and descending (documents of equal length in any order)
        assert sorted(items) == sorted((d, r) for d, r, _ in ref)
        docs = [d for i, (d, _) in enumerate(items) if i == 0 or items[i - 1][0] != d]
        assert len(docs) == len(set(docs)), "a document's tiles must be contiguous"
        nt = {d: sum(1 for dd, _ in items if dd == d) for d in docs}
        assert all(nt[a] >= nt[b] for a, b in zip(docs, docs[1:])), "documents must not grow"
        for d in docs:
            rs = [r for dd, r in items if dd == d]
            assert rs == list(range(nt[d] - 1, -1, -1)), f"document {d}: tiles not descending"


@pytest.mark.parametrize("cu", [[0, 500, 400, 1000], [0, 100, 1001], [5, 100, 1000], [0, 100, 999]])
def test_broken_cu_seqlens_writes_nothing(cu):
    H, T, D, sb = 1, 1000, 64, 64
    cu = np.asarray(cu, dtype=np.int32)
    nd = len(cu) - 1
    z8 = torch.zeros((H, T, D), dtype=torch.uint8, device="cuda")
    zd = torch.ones((H, ov.num_slots(T, nd, sb)), dtype=torch.float32, device="cuda")
    o = torch.full((H, T, D), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, T), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.zeros(fa.attn_fp8_varlen_workspace_bytes(T, nd), dtype=torch.uint8, device="cuda")
    fa.attn_fp8_fwd_varlen(z8, z8, z8, zd, zd, zd, dev(cu), scale_block=sb, causal=True, out=(o, lse), workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy().view(np.int32)
    assert w[0] == 0 and w[1] == 1
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)


# ---- full size: the packed workloads the benchmark times (T = 131072, 16 heads, d = 128)

@pytest.fixture(scope="module")
def packed_cache():
    return {}


@pytest.mark.slow
@pytest.mark.parametrize("name", ["packed_skewed_causal", "packed_long_causal", "packed_skewed"])
def test_packed_workload_parity(name, packed_cache):
    w = workloads.PACKED_WORKLOADS[name]
    cu = w.cu_seqlens()
    nd = len(cu) - 1
    key = (w.kind, w.H, w.T, w.D, w.data_seed)
    if key not in packed_cache:
        print(f"\n[{name}] generating {w.H}x{w.T}x{w.D}", flush=True)
        packed_cache.clear()
        packed_cache[key] = workloads.generate_packed_workload(w)
    q, k, v = packed_cache[key]
    print(f"[{name}] {nd} documents, lengths {int(np.diff(cu).min())} .. {int(np.diff(cu).max())}", flush=True)
    cu_d = dev(cu)
    print(f"[{name}] quantise + attention on the GPU", flush=True)
    qq = fa.quantize_qkv_fp8_varlen(dev(q), dev(k), dev(v), cu_d, scale_block=w.scale_block, hadamard=w.hadamard,
                                    seed=w.sign_seed)
    o, lse = fa.attn_fp8_fwd_varlen(*qq, cu_d, scale_block=w.scale_block, hadamard=w.hadamard, causal=w.causal)
    torch.cuda.synchronize()
    lens = np.diff(cu)
    docs = sorted({0, nd - 1, int(np.argmax(lens)), int(np.argmin(lens))})
    used = _used_slots(cu, w.T, w.scale_block)
    for h in sorted({0, w.H - 1}):
        sl = slice(h, h + 1)
        ref = ov.quantize_qkv_varlen(q[sl], k[sl], v[sl], cu, w.scale_block, w.hadamard, w.sign_seed)
        for g, r, nm in zip((host(t[sl]) for t in qq), ref, ("q8", "k8", "v8", "qd", "kd", "vd")):
            if r.dtype == np.uint8:
                assert np.array_equal(g, r), f"{name} head {h}: {nm}"
            else:
                assert np.array_equal(g[:, used].view(np.uint32), r[:, used].view(np.uint32)), f"{name} head {h}: {nm}"
        rows = np.concatenate([int(cu[d]) + np.array([r for r in sample_rows(int(lens[d]), 8, seed=d)
                                                      if r < lens[d]], dtype=np.int64) for d in docs])
        bars = ov.emulated_fp8_attention_varlen_bars(*ref, cu, w.scale_block, w.hadamard, w.causal, rows=rows)
        og, lg = host(o[sl])[:, rows], host(lse[sl])[:, rows]
        check_fp8_vs_e1(og, lg, bars, tag=f"[{name}] head {h} documents {docs}")
        orf, _ = ov.reference_attention_varlen(q[sl], k[sl], v[sl], cu, w.causal, rows=rows)
        print(f"[{name}] head {h}: vs FP64 rmse {rms(og - orf):.3e}", flush=True)
