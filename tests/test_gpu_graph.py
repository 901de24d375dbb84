"""Every entry point captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: each replay, with eager work and synchronisations between replays,
must reproduce the eager call's outputs bit for bit (the kernels are
deterministic: fixed reduction orders, split-k partials summed in split
order).  The library records kernel launches only -- no memset or copy nodes
-- so nothing in a replay depends on state left by an earlier one except the
caller's buffers."""
import numpy as np
import pytest
import torch

import quantized_linear_layer_amd as qll
import synth
from gpu_util import dev, empty

pytestmark = pytest.mark.gpu


def _setup():
    rng = np.random.default_rng(20261202)
    bufs, calls = {}, []

    # Q4_0 x Q8_0: decode GEMV (k = 4096, n = 300) and a prefill GEMM whose
    # plan has two k-splits (so the prepass, the GEMM and the split sum run)
    for tag, (m, n, k) in {"gemv": (1, 300, 4096), "gemm": (130, 257, 1024)}.items():
        codes, d_bits = synth.q4_0_weights(rng, n, k)
        w = empty(n * (k // 32) * 18)
        qll.qll_pack_q4_0(dev(codes), dev(np.asarray(d_bits, np.uint16).view(np.int16)), w, n, k)
        x = dev(synth.normal_f32(rng, (m, k)))
        xq = empty(m * (k // 32) * 34)
        y = empty(m * n, torch.float32)
        bufs[f"q4_{tag}_xq"], bufs[f"q4_{tag}_y"] = xq, y
        calls.append(lambda x=x, xq=xq, m=m, k=k: qll.qll_quantize_q8_0(x, xq, m, k))
        if m == 1:
            calls.append(lambda w=w, xq=xq, y=y, n=n, k=k: qll.qll_q4_0_q8_0_gemv(w, xq, y, n, k))
        else:
            need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, n, k)
            ws = empty(need)
            calls.append(lambda w=w, xq=xq, y=y, m=m, n=n, k=k, ws=ws: qll.qll_q4_0_q8_0_gemm(w, xq, y, m, n, k,
                                                                                           ws=ws))

    # f32: the m = 1 GEMV (partials + finish) and a small GEMM
    for tag, (m, n, k) in {"sgemv": (1, 1024, 2048), "sgemm": (96, 160, 64)}.items():
        a = dev(synth.uniform_f32(rng, (m, k)))
        b = dev(synth.uniform_f32(rng, (k, n)))
        c = empty(m * n, torch.float32)
        need = qll.qll_workspace_bytes(qll.QLL_OP_SGEMM, m, n, k)
        ws = empty(need) if need else None
        bufs[f"f32_{tag}_c"] = c
        calls.append(lambda a=a, b=b, c=c, m=m, n=n, k=k, ws=ws: qll.qll_sgemm(a, b, c, m, n, k, ws=ws))

    # ternary: int8 row quantization, GEMV and GEMM
    n, k = 640, 2560
    codes = synth.ternary_codes(rng, n, k)
    tw = empty(n * (k // 16), torch.int32)
    qll.qll_pack_ternary(dev(codes), tw, n, k)
    for m in (1, 64):
        x = dev(synth.normal_f32(rng, (m, k)))
        q = empty(m * k, torch.int8)
        s = empty(m, torch.float32)
        t = empty(m, torch.int32)
        y = empty(m * n, torch.float32)
        bufs.update({f"ter{m}_q": q, f"ter{m}_s": s, f"ter{m}_t": t, f"ter{m}_y": y})
        calls.append(lambda x=x, q=q, s=s, t=t, m=m: qll.qll_quantize_i8_rows(x, q, s, t, m, k))
        if m == 1:
            calls.append(lambda q=q, s=s, t=t, y=y: qll.qll_ternary_gemv(tw, 0.75, q, s, t, y, n, k))
        else:
            calls.append(lambda q=q, s=s, t=t, y=y, m=m: qll.qll_ternary_gemm(tw, 0.75, q, s, t, y, m, n, k))
    return bufs, calls


def _snapshot(bufs):
    torch.cuda.synchronize()
    return {name: b.cpu().numpy().view(np.uint8).copy() for name, b in bufs.items()}


def test_graph_replays_match_eager(qll_gpu):
    bufs, calls = _setup()
    for c in calls:
        c()
    eager = _snapshot(bufs)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in calls:
            c()
    for replay in range(4):
        for b in bufs.values():                          # eager work between replays
            b.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        got = _snapshot(bufs)
        for name in bufs:
            assert np.array_equal(got[name], eager[name]), f"replay {replay}: {name} differs from the eager call"
    del graph
    # the eager path still works after the graph is gone
    for c in calls:
        c()
    again = _snapshot(bufs)
    for name in bufs:
        assert np.array_equal(again[name], eager[name]), f"eager after graph: {name}"
