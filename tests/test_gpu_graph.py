"""Every compute entry point, on each of its kernel paths, captured into a
HIP graph (torch.cuda.CUDAGraph) and replayed: each replay, with eager work and synchronisations between replays,
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

    # Q4_0 at small m: the int8 matrix-core kernel (m = 4, m = 16), the
    # GEMV-style kernel by groups of eight rows (m = 12 with three blocks per
    # row), and the quantize-fused entry (m = 3)
    for tag, (m, n, k) in {"m4": (4, 200, 1024), "m16": (16, 300, 2048), "m12odd": (12, 140, 96)}.items():
        codes, d_bits = synth.q4_0_weights(rng, n, k)
        w = empty(n * (k // 32) * 18)
        qll.qll_pack_q4_0(dev(codes), dev(np.asarray(d_bits, np.uint16).view(np.int16)), w, n, k)
        xq = empty(m * (k // 32) * 34)
        qll.qll_quantize_q8_0(dev(synth.normal_f32(rng, (m, k))), xq, m, k)
        y = empty(m * n, torch.float32)
        need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, n, k)
        ws = empty(need) if need else None
        bufs[f"q4_{tag}_y"] = y
        calls.append(lambda w=w, xq=xq, y=y, m=m, n=n, k=k, ws=ws: qll.qll_q4_0_q8_0_gemm(w, xq, y, m, n, k,
                                                                                       ws=ws))
        if tag == "m4":
            xf = dev(synth.normal_f32(rng, (3, k)))
            yf = empty(3 * n, torch.float32)
            bufs["q4_fused_y"] = yf
            calls.append(lambda w=w, xf=xf, yf=yf, n=n, k=k: qll.qll_q4_0_q8_0_gemv_f32(w, xf, yf, 3, n, k))
            yfw = empty(3 * n, torch.float32)
            fws = empty(qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_GEMV_F32, 3, n, k))
            bufs["q4_fused_ws_y"] = yfw
            calls.append(lambda w=w, xf=xf, yfw=yfw, n=n, k=k, fws=fws: qll.qll_q4_0_q8_0_gemv_f32(w, xf, yfw, 3, n,
                                                                                                  k, ws=fws))

    # weights repacked at load time (Q4_0 and Q8_0) and the Q8_0-weight GEMV
    m, n, k = 64, 200, 512
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    w4 = empty(n * (k // 32) * 18)
    qll.qll_pack_q4_0(dev(codes), dev(np.asarray(d_bits, np.uint16).view(np.int16)), w4, n, k)
    w4p = empty(qll.qll_q4_0_repacked_bytes(n, k))
    qll.qll_q4_0_repack(w4, w4p, n, k)
    w8 = empty(n * (k // 32) * 34)
    qll.qll_quantize_q8_0(dev(synth.normal_f32(rng, (n, k))), w8, n, k)
    w8p = empty(qll.qll_q8_0_repacked_bytes(n, k))
    qll.qll_q8_0_repack(w8, w8p, n, k)
    xq = empty(m * (k // 32) * 34)
    qll.qll_quantize_q8_0(dev(synth.normal_f32(rng, (m, k))), xq, m, k)
    for tag, fn, op in (("q4r", qll.qll_q4_0_repacked_q8_0_gemm, qll.QLL_OP_Q4_0_REPACKED_GEMM),
                        ("q8r", qll.qll_q8_0_repacked_q8_0_gemm, qll.QLL_OP_Q8_0_REPACKED_GEMM)):
        wp = w4p if tag == "q4r" else w8p
        y = empty(m * n, torch.float32)
        ws = empty(max(16, qll.qll_workspace_bytes(op, m, n, k)))
        bufs[f"{tag}_y"] = y
        calls.append(lambda fn=fn, wp=wp, y=y, ws=ws, xq=xq, m=m, n=n, k=k: fn(wp, xq, y, m, n, k, ws=ws))
    y8 = empty(n, torch.float32)
    bufs["q8w_gemv_y"] = y8
    calls.append(lambda w8=w8, xq=xq, y8=y8, n=n, k=k: qll.qll_q8_0_q8_0_gemv(w8, xq, y8, n, k))
    # the decode GEMV on the decode-packed Q4_0 layout
    w4d = empty(qll.qll_q4_0_decode_packed_bytes(n, k))
    qll.qll_q4_0_decode_pack(w4, w4d, n, k)
    y4d = empty(n, torch.float32)
    bufs["q4_packed_gemv_y"] = y4d
    calls.append(lambda w4d=w4d, xq=xq, y4d=y4d, n=n, k=k: qll.qll_q4_0_decode_packed_q8_0_gemv(w4d, xq, y4d, n, k))

    # transposed-B: every weight type at m = 1 and m = 64, on the f32 matrix
    # core (no workspace) and on the bf16 one (a workspace); and the plain
    # f32 GEMM on the bf16 matrix core
    m, n, k = 64, 144, 320
    x = dev(synth.normal_f32(rng, (m, k)))
    w32 = synth.uniform_f32(rng, (n, k))
    for dt, code in (("f32", qll.QLL_DTYPE_F32), ("bf16", qll.QLL_DTYPE_BF16), ("f16", qll.QLL_DTYPE_F16)):
        wt = dev(w32)
        wt = wt if dt == "f32" else wt.to(torch.bfloat16 if dt == "bf16" else torch.float16)
        op = {"f32": qll.QLL_OP_GEMM_NT_F32, "bf16": qll.QLL_OP_GEMM_NT_BF16, "f16": qll.QLL_OP_GEMM_NT_F16}[dt]
        for core in ((False, True) if dt != "bf16" else (True,)):
            y = empty(m * n, torch.float32)
            ws = empty(max(16, qll.qll_workspace_bytes(op, m, n, k))) if core else None
            bufs[f"nt_{dt}_{core}_y"] = y
            calls.append(lambda wt=wt, code=code, y=y, ws=ws, x=x, m=m, n=n, k=k: qll.qll_gemm_nt(x, wt, code, y, m, n,
                                                                                              k, ws=ws))
        y1 = empty(n, torch.float32)
        bufs[f"nt_{dt}_gemv_y"] = y1
        calls.append(lambda wt=wt, code=code, y1=y1, x=x, n=n, k=k: qll.qll_gemm_nt(x[:1], wt, code, y1, 1, n, k))
    b = dev(synth.uniform_f32(rng, (k, n)))
    c = empty(m * n, torch.float32)
    wsc = empty(qll.qll_workspace_bytes(qll.QLL_OP_SGEMM_BF16, m, n, k))
    bufs["sgemm_core_c"] = c
    calls.append(lambda x=x, b=b, c=c, m=m, n=n, k=k, wsc=wsc: qll.qll_sgemm(x, b, c, m, n, k, ws=wsc))

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
