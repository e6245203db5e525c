"""HIP graph capture of the FP8 path ("FLAMIA", F. System Integration: scales and
work lists stay on the GPU, so a call is captured without host
synchronisation and its replay equals eager execution bit for bit).

Every entry point queues only its own kernels on the caller's stream (no
allocation, no memset, no host copy), so a captured quantise + attention
(dense, packed documents, decode) replays to the same bits as an eager call.
Each test replays several times, with eager work and synchronisations in
between, and also replays after new values are copied into the captured input
buffers.
"""

import numpy as np
import pytest
import torch

import fp8_attention_forward_amd as fa
import workloads
from tests.gpu_common import dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _replays_match(graph, outputs, eager, refresh=None, n=3):
    """Replay `graph` n times (eager work in between) and compare every output
    with a fresh eager run; `refresh` may rewrite the captured inputs first."""
    for i in range(n):
        if refresh is not None and i == n - 1:
            refresh()
        ref = [t.clone() for t in eager()]
        torch.cuda.synchronize()
        for t in outputs:
            t.fill_(-7)                      # (a fill kernel: no memset node in the graph)
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, ref):
            assert torch.equal(got, want), f"replay {i} differs from eager"


@pytest.mark.parametrize("causal", [False, True])
def test_dense_quantise_and_attention_graph(causal):
    B, H, N, D, sb = 1, 4, 1000, 128, 128
    q, k, v = (dev(x) for x in workloads.generate("outlier", B, H, N, D, 71))
    qo = fa.quantize_qkv_fp8(q, k, v, scale_block=sb)
    o, lse = fa.attn_fp8_fwd(*qo, scale_block=sb, causal=causal)
    o_s, l_s = torch.empty_like(o), torch.empty_like(lse)
    torch.cuda.synchronize()

    def eager():
        fa.quantize_qkv_fp8(q, k, v, scale_block=sb, out=qo)
        fa.attn_fp8_fwd(*qo, scale_block=sb, causal=causal, out=(o, lse))
        fa.attn_fp8_fwd(*qo, scale_block=sb, causal=causal, out=(o_s, l_s), exp2="schraudolph")
        return o, lse, o_s, l_s

    eager()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            eager()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    captured = [o, lse, o_s, l_s]
    snapshot = [t.clone() for t in captured]

    def eager_copy():
        eager()
        return [t.clone() for t in captured]

    new = [dev(x) for x in workloads.generate("iid", B, H, N, D, 72)]

    def refresh():
        for dst, src in zip((q, k, v), new):
            dst.copy_(src)

    _replays_match(g, captured, eager_copy, refresh)
    assert not torch.equal(snapshot[0], o)          # the last replay saw the new inputs


def test_packed_documents_graph():
    H, D, sb = 2, 128, 128
    cu_np = np.array([0, 1, 300, 300, 777, 1500], dtype=np.int32)
    T = int(cu_np[-1])
    q, k, v = (dev(x) for x in workloads.generate_packed("outlier", H, T, D, 73))
    cu = dev(cu_np)
    ws = torch.empty(fa.attn_fp8_varlen_workspace_bytes(T, len(cu_np) - 1), dtype=torch.uint8, device="cuda")
    qo = fa.quantize_qkv_fp8_varlen(q, k, v, cu, scale_block=sb)
    o, lse = fa.attn_fp8_fwd_varlen(*qo, cu, scale_block=sb, causal=True, workspace=ws)
    torch.cuda.synchronize()

    def eager():
        fa.quantize_qkv_fp8_varlen(q, k, v, cu, scale_block=sb, out=qo)
        fa.attn_fp8_fwd_varlen(*qo, cu, scale_block=sb, causal=True, out=(o, lse), workspace=ws)
        return [o.clone(), lse.clone()]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fa.quantize_qkv_fp8_varlen(q, k, v, cu, scale_block=sb, out=qo)
            fa.attn_fp8_fwd_varlen(*qo, cu, scale_block=sb, causal=True, out=(o, lse), workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    _replays_match(g, [o, lse], eager)


def test_decode_graph():
    B, Hq, Hkv, Sq, N, D, sb = 3, 8, 2, 1, 2000, 128, 128
    q, k, v = workloads.generate_decode("iid", B, Hq, Hkv, Sq, N, D, 74)
    _, k8, v8, _, kd, vd = fa.quantize_qkv_fp8(dev(k), dev(k), dev(v), scale_block=sb)
    q8, _, _, qd, _, _ = fa.quantize_qkv_fp8(dev(q), dev(q), dev(q), scale_block=sb)
    sl = dev(np.array([2000, 17, 1234], dtype=np.int32))
    ws = torch.empty(fa.attn_fp8_decode_workspace_bytes(B, Hq, Hkv, Sq, N, D), dtype=torch.uint8, device="cuda")
    o, lse = fa.attn_fp8_decode(q8, qd, k8, v8, kd, vd, sl, scale_block=sb, workspace=ws)
    torch.cuda.synchronize()

    def eager():
        fa.attn_fp8_decode(q8, qd, k8, v8, kd, vd, sl, scale_block=sb, workspace=ws, out=(o, lse))
        return [o.clone(), lse.clone()]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fa.attn_fp8_decode(q8, qd, k8, v8, kd, vd, sl, scale_block=sb, workspace=ws, out=(o, lse))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def refresh():
        sl.copy_(dev(np.array([999, 2000, 64], dtype=np.int32)))     # new lengths, read on the device

    _replays_match(g, [o, lse], eager, refresh)
