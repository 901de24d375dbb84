"""Benchmark of the quantized linear layer hot path on one MI355X.

One step is one pass of every operation of the path at its full workload
size, on inputs already resident in HBM:
  * the Q4_0 x Q8_0 GEMV of the 512 x 512 layer (m = 1);
  * Q8_0 quantization of the decode activation and Q4_0 x Q8_0 decode GEMV
    (m = 1) on the four 8B-class linear shapes (k, n) = (4096, 14336),
    (14336, 4096), (4096, 4096), (4096, 128256);
  * Q8_0 quantization of the prefill activations and the Q4_0 x Q8_0 prefill
    GEMM (m = 512) on the same four shapes and weights;
  * the f32 GEMM 4096^3 and the f32 GEMV 4096 x 4096;
  * the BitNet ternary layer 2560 -> 6912: int8 row quantization, GEMV (m = 1)
    and GEMM (m = 64).
Measured in the same run, outside the step: the Q4_0 prefill GEMM on the same
weights repacked at load time into the matrix core's 6-bit operand form; the
four shapes with Q8_0 weights (decode GEMV, prefill GEMM on repacked
weights); the f32 GEMV and GEMM in the transposed-B orientation (W = B^T
stored [n][k]) with f32, bf16 and f16 weights; the (4096 -> 14336) layer over
prompt lengths m = 1, 2, 4, 8, 16, 32, 64, 129, 256, 512; and the
quantize-fused decode entry against quantize + decode at m = 1 and 8.
Decode weights rotate through enough device copies (>= 1 GiB per shape) that
no decode GEMV reads its weights from the 256 MiB Infinity Cache.

Timing uses HIP events recorded on the stream the library launches on
(torch's current stream).  `ms_per_step` is the wall time of the timed steps,
each op bracketed by its own event pair.  An event pair around one lone
launch also holds the event and dispatch latency (2-3 us, a third of a small
decode GEMV), so each op's average launch duration is taken from R
back-to-back launches captured once into a HIP graph (the decode ops still
rotating through their weight copies) and replayed between one event pair,
R chosen for about a millisecond per replay, with at least 7 replays and 200
launches per op.

Output: the per-kernel table goes to stderr (and to --kernels-out), and stdout
ends with ONE short JSON line: `value` is the Q4_0 x Q8_0 decode GEMV
bandwidth over the four shapes (algorithmic bytes / summed average launch
duration); `roofline` describes the kernel with the largest share of the
step; `per_format` holds decode GB/s and prefill TOPS of every format with
their fractions of the MI355X peaks; `rows` the per-workload times;
`cpu_baseline` times the oracle (the test suite's plain C reference, never
tuned) on every workload on the host's physical cores; `device` records the
GPU, the bandwidth of a plain 1 GiB device copy (a second HBM denominator)
and a hash of the kernel sources.  A row whose launch times vary by more than
8% (coefficient of variation) is flagged noisy.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "i8": 5000.0, "f32": 157.3, "bf6": 10100.0}
METRIC = "decode GEMV HBM GB/s (% of peak) + prefill GEMM TOPS (% MFMA peak) per format"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="bound on the oracle's CPU sample")
    p.add_argument("--only", default="", help="comma-separated op-name prefixes to run (profiling)")
    p.add_argument("--kernels-out", default="", help="also write the per-kernel table (JSON) to this file")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy per step (counter calibration)")
    return p.parse_args()


# Operations of the rows beyond the hot path's core (small-m, repacked weights,
# Q8_0 weights, transposed-B): timed the same way, but not part of a step.
NOISY_CV = 0.08  # coefficient of variation above which a row is flagged noisy
EXTRA_PREFIXES = ("q4r_gemm", "q4p_gemv", "q8w_gemv", "q8r_gemm", "nt_", "sgemm_core", "msweep_", "f1_")
M_SWEEP = (1, 2, 4, 8, 16, 32, 64, 129, 256, 512)  # prompt lengths straddling the tile edges


class Op:
    def __init__(self, name, fmt, kind, fn, nbytes, flops, bound, peak_key=None):
        self.name, self.fmt, self.kind, self.fn = name, fmt, kind, fn
        self.nbytes, self.flops, self.bound, self.peak_key = nbytes, flops, bound, peak_key
        self.in_step = not name.startswith(EXTRA_PREFIXES)
        self.times_ms = []  # event pair around the op's single launch in each step
        self.batch_ms = []  # per launch, from runs of back-to-back launches
        self.reps = 1

    def roofline(self, ms):
        if self.bound == "hbm":
            achieved = self.nbytes / (ms * 1e-3) / 1e9
            return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS}
        achieved = self.flops / (ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[self.peak_key]
        return {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s" if self.peak_key != "i8"
                else "TOP/s", "frac": achieved / peak}


def q8_0_block_bytes(np, codes, d_bits):
    """The raw Q8_0 weight draws laid out as block_q8_0 records: little-endian
    binary16 d, then the block's 32 int8 codes (34 bytes per block)."""
    n, k = codes.shape
    nb = k // 32
    blk = np.empty((n, nb, 34), np.uint8)
    blk[:, :, 0:2] = np.ascontiguousarray(d_bits.astype("<u2")).view(np.uint8).reshape(n, nb, 2)
    blk[:, :, 2:] = codes.reshape(n, nb, 32).view(np.uint8)
    return blk.reshape(-1)


def build_ops(qll, synth, torch, np, dev, only):
    ops = []
    keep = [s for s in only.split(",") if s]

    def want(name):
        return not keep or any(name.startswith(s) for s in keep)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    gib = 1 << 30
    step_ref = {"i": 0}

    # ---------------------------------------------------------------- Q4_0 x Q8_0
    for s, (k, n) in enumerate(synth.SHAPES_8B):
        need_dec = want(f"q4_gemv_{s}") or want(f"q8_quant_decode_{s}") or want(f"q4p_gemv_{s}")
        need_pre = want(f"q4_gemm_{s}") or want(f"q8_quant_prefill_{s}") or want(f"q4r_gemm_{s}")
        if not (need_dec or need_pre):
            continue
        codes, d_bits, x = synth.q4_decode(s)
        w0 = torch.empty(n * (k // 32) * 18, dtype=torch.uint8, device=dev)
        qll.qll_pack_q4_0(to_dev(codes), to_dev(d_bits.view(np.int16)), w0, n, k)
        del codes, d_bits
        wbytes = w0.numel()
        if need_dec:
            copies = [w0] + [w0.clone() for _ in range(max(1, -(-gib // wbytes)) - 1)]
            xd = to_dev(x)
            xqd = torch.empty((k // 32) * 34, dtype=torch.uint8, device=dev)
            yd = torch.empty(n, dtype=torch.float32, device=dev)
            if want(f"q8_quant_decode_{s}"):
                ops.append(Op(f"q8_quant_decode_{s}", "q4_0", "quant",
                              lambda xd=xd, xqd=xqd, k=k: qll.qll_quantize_q8_0(xd, xqd, 1, k),
                              4 * k + (k // 32) * 34, 0, "hbm"))
            if want(f"q4_gemv_{s}"):
                ops.append(Op(f"q4_gemv_{s}", "q4_0", "decode",
                              lambda c=copies, xqd=xqd, yd=yd, n=n, k=k: qll.qll_q4_0_q8_0_gemv(
                                  c[step_ref["i"] % len(c)], xqd, yd, n, k),
                              wbytes + (k // 32) * 34 + 4 * n, 2 * n * k, "hbm"))
            if want(f"q4p_gemv_{s}"):
                # the same weights in the decode-packed layout, as many rotating copies
                pbytes = qll.qll_q4_0_decode_packed_bytes(n, k)
                pcopies = []
                for c0 in copies:
                    wpk = torch.empty(pbytes, dtype=torch.uint8, device=dev)
                    qll.qll_q4_0_decode_pack(c0, wpk, n, k)
                    pcopies.append(wpk)
                qll.qll_quantize_q8_0(xd, xqd, 1, k)
                ypk = torch.empty(n, dtype=torch.float32, device=dev)
                ops.append(Op(f"q4p_gemv_{s}", "q4_0_decode_packed", "decode",
                              lambda c=pcopies, xqd=xqd, ypk=ypk, n=n, k=k: qll.qll_q4_0_decode_packed_q8_0_gemv(
                                  c[step_ref["i"] % len(c)], xqd, ypk, n, k),
                              pbytes + (k // 32) * 34 + 4 * n, 2 * n * k, "hbm"))
        if need_pre:
            m = 512
            xp = to_dev(synth.q4_prefill_x(s))
            xqp = torch.empty(m * (k // 32) * 34, dtype=torch.uint8, device=dev)
            yp = torch.empty(m * n, dtype=torch.float32, device=dev)
            if want(f"q8_quant_prefill_{s}"):
                ops.append(Op(f"q8_quant_prefill_{s}", "q4_0", "quant",
                              lambda xp=xp, xqp=xqp, k=k: qll.qll_quantize_q8_0(xp, xqp, 512, k),
                              4 * m * k + m * (k // 32) * 34, 0, "hbm"))
            if want(f"q4_gemm_{s}"):
                # the prefill GEMM needs quantized activations even when profiled alone
                qll.qll_quantize_q8_0(xp, xqp, m, k)
                need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, n, k)
                wsp = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
                ops.append(Op(f"q4_gemm_{s}", "q4_0", "prefill",
                              lambda w0=w0, xqp=xqp, yp=yp, n=n, k=k, wsp=wsp: qll.qll_q4_0_q8_0_gemm(
                                  w0, xqp, yp, 512, n, k, ws=wsp),
                              wbytes + m * (k // 32) * 34 + 4 * m * n, 2 * m * n * k, "mfma", "f16"))
            if want(f"q4r_gemm_{s}"):
                qll.qll_quantize_q8_0(xp, xqp, m, k)
                wp = torch.empty(qll.qll_q4_0_repacked_bytes(n, k), dtype=torch.uint8, device=dev)
                qll.qll_q4_0_repack(w0, wp, n, k)
                need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_REPACKED_GEMM, m, n, k)
                wsr = torch.empty(need, dtype=torch.uint8, device=dev)
                yr = torch.empty(m * n, dtype=torch.float32, device=dev)
                ops.append(Op(f"q4r_gemm_{s}", "q4_0_repacked", "prefill",
                              lambda wp=wp, xqp=xqp, yr=yr, n=n, k=k, wsr=wsr: qll.qll_q4_0_repacked_q8_0_gemm(
                                  wp, xqp, yr, 512, n, k, ws=wsr),
                              wp.numel() + m * (k // 32) * 34 + 4 * m * n, 2 * m * n * k, "mfma", "bf6"))
        if need_dec and want(f"q4_gemv_{s}") and not want(f"q8_quant_decode_{s}"):
            qll.qll_quantize_q8_0(xd, xqd, 1, k)

    # ---------------------------------------------------------------- Q4_0 512 x 512 layer (m = 1)
    if want("q4_gemv_small"):
        codes, d_bits, x = synth.q4_small()
        n1, k1 = codes.shape
        w1 = torch.empty(n1 * (k1 // 32) * 18, dtype=torch.uint8, device=dev)
        qll.qll_pack_q4_0(to_dev(codes), to_dev(d_bits.view(np.int16)), w1, n1, k1)
        xq1 = torch.empty((k1 // 32) * 34, dtype=torch.uint8, device=dev)
        qll.qll_quantize_q8_0(to_dev(x), xq1, 1, k1)
        y1 = torch.empty(n1, dtype=torch.float32, device=dev)
        ops.append(Op("q4_gemv_small", "q4_0_small", "decode",
                      lambda: qll.qll_q4_0_q8_0_gemv(w1, xq1, y1, n1, k1),
                      w1.numel() + xq1.numel() + 4 * n1, 2 * n1 * k1, "hbm"))

    # ---------------------------------------------------------------- prompt-length sweep, fused decode
    # (4096 -> 14336): m over prompt lengths that straddle the kernels' row
    # tiles (m = 1 GEMV, 2..32 the small-m kernels, which read the weights
    # once, up to 64 by groups of 32 rows, above it the 128-row GEMM), and the
    # quantize-fused decode entry
    # against the quantize + decode pair at m = 1 and m = 8 on every 8B-class
    # shape.
    for s, (k, n) in enumerate(synth.SHAPES_8B):
        sweep = s == 0 and any(want(f"msweep_q4_m{m}") for m in M_SWEEP)
        fused = any(want(f"f1_{kind}_m{m}_{s}") for kind in ("fused", "pair") for m in (1, 8))
        if not (sweep or fused):
            continue
        codes, d_bits, _ = synth.q4_decode(s)
        w0 = torch.empty(n * (k // 32) * 18, dtype=torch.uint8, device=dev)
        qll.qll_pack_q4_0(to_dev(codes), to_dev(d_bits.view(np.int16)), w0, n, k)
        del codes, d_bits
        wbytes = w0.numel()
        copies = [w0] + [w0.clone() for _ in range(max(1, -(-gib // wbytes)) - 1)]
        xall = to_dev(synth.q4_prefill_x(s))
        ms = [m for m in M_SWEEP if sweep and want(f"msweep_q4_m{m}")]
        for m in ms:
            xqm = torch.empty(m * (k // 32) * 34, dtype=torch.uint8, device=dev)
            qll.qll_quantize_q8_0(xall[:m].contiguous(), xqm, m, k)
            ym = torch.empty(m * n, dtype=torch.float32, device=dev)
            need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, n, k)
            wsm = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
            ops.append(Op(f"msweep_q4_m{m}", "q4_0_msweep", "sweep",
                          lambda c=copies, xqm=xqm, ym=ym, m=m, n=n, k=k, wsm=wsm: qll.qll_q4_0_q8_0_gemm(
                              c[step_ref["i"] % len(c)], xqm, ym, m, n, k, ws=wsm),
                          wbytes + m * (k // 32) * 34 + 4 * m * n, 2 * m * n * k, "hbm" if m <= 64 else "mfma",
                          None if m <= 64 else "f16"))
        for m in ((1, 8) if fused else ()):
            xm = xall[:m].contiguous()
            xqm = torch.empty(m * (k // 32) * 34, dtype=torch.uint8, device=dev)
            ym = torch.empty(m * n, dtype=torch.float32, device=dev)
            if want(f"f1_fused_m{m}_{s}"):
                need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_GEMV_F32, m, n, k)
                fws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
                ops.append(Op(f"f1_fused_m{m}_{s}", "q4_0_fused", "decode",
                              lambda c=copies, xm=xm, ym=ym, m=m, n=n, k=k, fws=fws: qll.qll_q4_0_q8_0_gemv_f32(
                                  c[step_ref["i"] % len(c)], xm, ym, m, n, k, ws=fws),
                              wbytes + 4 * m * k + 4 * m * n, 2 * m * n * k, "hbm"))
            if want(f"f1_pair_m{m}_{s}"):
                def pair(c=copies, xm=xm, xqm=xqm, ym=ym, m=m, n=n, k=k):
                    qll.qll_quantize_q8_0(xm, xqm, m, k)
                    qll.qll_q4_0_q8_0_gemm(c[step_ref["i"] % len(c)], xqm, ym, m, n, k)
                ops.append(Op(f"f1_pair_m{m}_{s}", "q4_0_pair", "decode", pair,
                              wbytes + 4 * m * k + 4 * m * n, 2 * m * n * k, "hbm"))

    # ---------------------------------------------------------------- Q8_0 weights
    for s, (k, n) in enumerate(synth.SHAPES_8B):
        need_dec, need_pre = want(f"q8w_gemv_{s}"), want(f"q8r_gemm_{s}")
        if not (need_dec or need_pre):
            continue
        codes, d_bits, x = synth.q8w_decode(s)
        w0 = to_dev(q8_0_block_bytes(np, codes, d_bits))
        del codes, d_bits
        wbytes = w0.numel()
        if need_dec:
            copies = [w0] + [w0.clone() for _ in range(max(1, -(-gib // wbytes)) - 1)]
            xqd = torch.empty((k // 32) * 34, dtype=torch.uint8, device=dev)
            qll.qll_quantize_q8_0(to_dev(x), xqd, 1, k)
            yd = torch.empty(n, dtype=torch.float32, device=dev)
            ops.append(Op(f"q8w_gemv_{s}", "q8_0", "decode",
                          lambda c=copies, xqd=xqd, yd=yd, n=n, k=k: qll.qll_q8_0_q8_0_gemv(
                              c[step_ref["i"] % len(c)], xqd, yd, n, k),
                          wbytes + (k // 32) * 34 + 4 * n, 2 * n * k, "hbm"))
        if need_pre:
            m = 512
            xqp = torch.empty(m * (k // 32) * 34, dtype=torch.uint8, device=dev)
            qll.qll_quantize_q8_0(to_dev(synth.q4_prefill_x(s)), xqp, m, k)
            wp = torch.empty(qll.qll_q8_0_repacked_bytes(n, k), dtype=torch.uint8, device=dev)
            qll.qll_q8_0_repack(w0, wp, n, k)
            wsr = torch.empty(qll.qll_workspace_bytes(qll.QLL_OP_Q8_0_REPACKED_GEMM, m, n, k), dtype=torch.uint8,
                              device=dev)
            yr = torch.empty(m * n, dtype=torch.float32, device=dev)
            ops.append(Op(f"q8r_gemm_{s}", "q8_0", "prefill",
                          lambda wp=wp, xqp=xqp, yr=yr, n=n, k=k, wsr=wsr: qll.qll_q8_0_repacked_q8_0_gemm(
                              wp, xqp, yr, 512, n, k, ws=wsr),
                          wp.numel() + m * (k // 32) * 34 + 4 * m * n, 2 * m * n * k, "mfma", "bf6"))
            if not need_dec:
                del w0

    # ---------------------------------------------------------------- f32
    if want("sgemm") or want("sgemv"):
        a, b, x = synth.f32_gemm()
        M = N = K = 4096
        bd = to_dev(b)
        if want("sgemm"):
            ad = to_dev(a)
            cd = torch.empty(M * N, dtype=torch.float32, device=dev)
            ops.append(Op("sgemm_4096", "f32", "prefill", lambda: qll.qll_sgemm(ad, bd, cd, M, N, K),
                          4 * (M * K + K * N + M * N), 2 * M * N * K, "mfma", "f32"))
        if want("sgemm_core"):
            # the same GEMM given a workspace: both operands split into three
            # exact bf16 parts on the bf16 matrix core (fraction of the bf16
            # peak; outside the step, which keeps the f32 matrix core)
            wsc = torch.empty(qll.qll_workspace_bytes(qll.QLL_OP_SGEMM_BF16, M, N, K), dtype=torch.uint8, device=dev)
            cdc = torch.empty(M * N, dtype=torch.float32, device=dev)
            ops.append(Op("sgemm_core_4096", "f32_core", "prefill",
                          lambda: qll.qll_sgemm(ad, bd, cdc, M, N, K, ws=wsc),
                          4 * (M * K + K * N + M * N), 2 * M * N * K, "mfma", "bf16"))
        if want("sgemv"):
            copies = [bd] + [bd.clone() for _ in range(max(1, -(-gib // (4 * K * N))) - 1)]
            xd = to_dev(x)
            yd = torch.empty(N, dtype=torch.float32, device=dev)
            ws = torch.empty(qll.qll_workspace_bytes(qll.QLL_OP_SGEMM, 1, N, K), dtype=torch.uint8, device=dev)
            ops.append(Op("sgemv_4096", "f32", "decode",
                          lambda c=copies: qll.qll_sgemm(xd, c[step_ref["i"] % len(c)], yd, 1, N, K, ws=ws),
                          4 * (K + K * N + N), 2 * N * K, "hbm"))
        del a, b, x

    # ---------------------------------------------------------------- transposed B (W [n][k]), f32/bf16/f16
    if want("nt_"):
        a, b, x = synth.f32_gemm()
        M = N = K = 4096
        wt = to_dev(np.ascontiguousarray(b.T))
        del b
        ad = to_dev(a) if want("nt_gemm") else None
        xd = to_dev(x)
        dts = (("f32", qll.QLL_DTYPE_F32, torch.float32), ("bf16", qll.QLL_DTYPE_BF16, torch.bfloat16),
               ("f16", qll.QLL_DTYPE_F16, torch.float16))
        for name, code, tdt in dts:
            w = wt if tdt == torch.float32 else wt.to(tdt)
            esz = w.element_size()
            if want(f"nt_gemv_{name}"):
                copies = [w] + [w.clone() for _ in range(max(1, -(-gib // (esz * N * K))) - 1)]
                yd = torch.empty(N, dtype=torch.float32, device=dev)
                ops.append(Op(f"nt_gemv_{name}_4096", f"{name}_nt", "decode",
                              lambda c=copies, yd=yd, code=code: qll.qll_gemm_nt(
                                  xd, c[step_ref["i"] % len(c)], code, yd, 1, N, K),
                              esz * N * K + 4 * K + 4 * N, 2 * N * K, "hbm"))
            if want(f"nt_gemm_{name}"):
                cd = torch.empty(M * N, dtype=torch.float32, device=dev)
                op_code = {"bf16": qll.QLL_OP_GEMM_NT_BF16, "f16": qll.QLL_OP_GEMM_NT_F16,
                           "f32": qll.QLL_OP_GEMM_NT_F32}[name]
                need = qll.qll_workspace_bytes(op_code, M, N, K)
                wsn = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
                bf = True
                # given a workspace, every weight type runs on the bf16 matrix
                # core (three, five or six bf16 MFMAs per product of an f32
                # activation for bf16, f16 or f32 weights): fraction of the
                # bf16 peak; the widened f32-matrix-core path is the plain
                # orientation's sgemm kernel
                ops.append(Op(f"nt_gemm_{name}_4096", f"{name}_nt", "prefill",
                              lambda w=w, cd=cd, code=code, wsn=wsn: qll.qll_gemm_nt(ad, w, code, cd, M, N, K, ws=wsn),
                              4 * M * K + esz * N * K + 4 * M * N, 2 * M * N * K, "mfma", "bf16" if bf else "f32"))
        del wt

    # ---------------------------------------------------------------- ternary
    if any(want(s) for s in ("i8_quant", "ternary")):
        codes, w_scale, x = synth.ternary_layer()
        n, k = codes.shape
        m = x.shape[0]
        tw0 = torch.empty(n * (k // 16), dtype=torch.int32, device=dev)
        qll.qll_pack_ternary(to_dev(codes), tw0, n, k)
        tcopies = [tw0] + [tw0.clone() for _ in range(max(1, -(-gib // (n * k // 4))) - 1)]
        xd = to_dev(x)
        q = torch.empty(m * k, dtype=torch.int8, device=dev)
        sc = torch.empty(m, dtype=torch.float32, device=dev)
        sm = torch.empty(m, dtype=torch.int32, device=dev)
        xd1 = to_dev(x[:1])
        q1 = torch.empty(k, dtype=torch.int8, device=dev)
        sc1 = torch.empty(4, dtype=torch.float32, device=dev)
        sm1 = torch.empty(4, dtype=torch.int32, device=dev)
        y1 = torch.empty(n, dtype=torch.float32, device=dev)
        ym = torch.empty(m * n, dtype=torch.float32, device=dev)
        qll.qll_quantize_i8_rows(xd, q, sc, sm, m, k)
        qll.qll_quantize_i8_rows(xd1, q1, sc1, sm1, 1, k)
        if want("i8_quant_decode"):
            ops.append(Op("i8_quant_decode", "ternary", "quant", lambda: qll.qll_quantize_i8_rows(
                xd1, q1, sc1, sm1, 1, k), 5 * k + 8, 0, "hbm"))
        if want("ternary_gemv"):
            ops.append(Op("ternary_gemv", "ternary", "decode", lambda: qll.qll_ternary_gemv(
                tcopies[step_ref["i"] % len(tcopies)], w_scale, q1, sc1, sm1, y1, n, k),
                n * k // 4 + k + 8 + 4 * n, 2 * n * k, "hbm"))
        if want("i8_quant_prefill"):
            ops.append(Op("i8_quant_prefill", "ternary", "quant", lambda: qll.qll_quantize_i8_rows(
                xd, q, sc, sm, m, k), 5 * m * k + 8 * m, 0, "hbm"))
        if want("ternary_gemm"):
            ops.append(Op("ternary_gemm", "ternary", "prefill", lambda: qll.qll_ternary_gemm(
                tw0, w_scale, q, sc, sm, ym, m, n, k),
                n * k // 4 + m * k + 8 * m + 4 * m * n, 2 * m * n * k, "mfma", "i8"))
    return ops, step_ref


def host_cpus():
    """(physical cores, logical CPUs, model name) of this process's affinity
    mask: logical CPUs that share a (package, core) pair are SMT siblings and
    count once."""
    cpus = sorted(os.sched_getaffinity(0))
    cores = set()
    for c in cpus:
        base = f"/sys/devices/system/cpu/cpu{c}/topology/"
        try:
            cores.add((open(base + "physical_package_id").read().strip(), open(base + "core_id").read().strip()))
        except OSError:
            cores.add(("?", str(c)))
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return len(cores), len(cpus), model


def cpu_baseline(synth, np, seconds):
    """The oracle (plain C: exact int32 block sums with f64 scaling, f64
    accumulation; never tuned) on every workload, on the physical cores of
    this process's affinity mask.  Small workloads run whole, repeated until
    a share of `seconds` has passed; the large GEMMs run on their first rows
    only (the oracle's cost is linear in the rows), which the entry states.
    `value` is the decode GEMV rate over the four 8B-class shapes, in the
    unit of the GPU's `value`."""
    import oracle as O
    phys, logical, model = host_cpus()
    O.set_num_threads(phys)

    def timed(fn, budget):
        t_total, passes = 0.0, 0
        while passes < 1 or (t_total < budget and passes < 10000):
            t0 = time.perf_counter()
            fn()
            t_total += time.perf_counter() - t0
            passes += 1
        return t_total / passes, passes

    out = {}

    def rec(name, per_pass_s, passes, nbytes=None, ops=None, sample="whole"):
        e = {"s": round(per_pass_s, 6), "passes": passes, "sample": sample}
        if nbytes is not None:
            e.update(value=round(nbytes / per_pass_s / 1e9, 3), unit="GB/s")
        else:
            e.update(value=round(ops / per_pass_s / 1e9, 3), unit="GOP/s")
        out[name] = e

    # 512 x 512 Q4_0 layer, m = 1
    codes, d_bits, x = synth.q4_small()
    w, xq = O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x)
    t, p = timed(lambda: O.q4_0_q8_0(w, xq, 1, 512, 512), 0.05 * seconds)
    rec("q4_gemv_512", t, p, nbytes=w.size + xq.size + 4 * 512)
    # 8B-class decode GEMVs (the four shapes together) and prefill GEMMs (first rows)
    dec, pre_rows = [], 4
    pre_ops, pre_t = 0, 0.0
    for s, (k, n) in enumerate(synth.SHAPES_8B):
        codes, d_bits, x = synth.q4_decode(s)
        w = O.pack_q4_0(codes, d_bits)
        del codes, d_bits
        dec.append((w, O.quantize_q8_0(x), n, k))
        xp = O.quantize_q8_0(synth.q4_prefill_x(s, m=pre_rows))
        t0 = time.perf_counter()
        O.q4_0_q8_0(w, xp, pre_rows, n, k)
        pre_t += time.perf_counter() - t0
        pre_ops += 2 * pre_rows * n * k
    dec_bytes = sum(w.size + xq.size + 4 * n for w, xq, n, k in dec)
    t, p = timed(lambda: [O.q4_0_q8_0(w, xq, 1, n, k) for w, xq, n, k in dec], 0.35 * seconds)
    rec("q4_gemv_8b", t, p, nbytes=dec_bytes)
    rec("q4_gemm_8b_m512", pre_t, 1, ops=pre_ops, sample=f"rows 0..{pre_rows - 1} of 512, four shapes")
    del dec
    # f32 GEMM 4096^3 (first rows) and GEMV 4096 x 4096
    a, b, x = synth.f32_gemm()
    rows = 16
    t0 = time.perf_counter()
    O.sgemm(a[:rows], b)
    rec("sgemm_4096", time.perf_counter() - t0, 1, ops=2 * rows * 4096 * 4096, sample=f"rows 0..{rows - 1} of 4096")
    t, p = timed(lambda: O.sgemm(x, b), 0.1 * seconds)
    rec("sgemv_4096", t, p, nbytes=4 * (4096 + 4096 * 4096 + 4096))
    del a, b
    # BitNet ternary 2560 -> 6912, m = 1 and m = 64 (quantization included)
    codes, w_scale, x = synth.ternary_layer()
    n, k = codes.shape
    words = O.pack_ternary(codes)

    def tern(xr):
        q, sc, sm = O.quantize_i8_rows(xr)
        O.ternary(words, w_scale, q, sc, sm, n, k)

    t, p = timed(lambda: tern(x[:1]), 0.1 * seconds)
    rec("ternary_m1", t, p, nbytes=words.size * 4 + 4 * k + 4 * n)
    t, p = timed(lambda: tern(x), 0.1 * seconds)
    rec("ternary_m64", t, p, ops=2 * 64 * n * k)
    return {"value": out["q4_gemv_8b"]["value"], "unit": "GB/s", "cores": phys, "logical_cpus": logical,
            "cpu_model": model, "kind": "oracle",
            "sample": "the oracle on every workload on the physical cores; GEMMs on their first rows (stated per "
                      "config); value = Q4_0 x Q8_0 decode GEMV over the four 8B-class shapes",
            "configs": out}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by output rows across GPUs; the library runs on one GPU).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import quantized_linear_layer_amd as qll
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qll.load()
    print("bench: setting up inputs", file=sys.stderr, flush=True)
    ops, step_ref = build_ops(qll, synth, torch, np, dev, args.only)
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        ops.append(Op("copy_1gib", "calibration", "copy", lambda: dst.copy_(src), 2 * src.numel() * 4, 0, "hbm"))
    torch.cuda.synchronize()
    print(f"bench: {len(ops)} ops per step; warmup {args.warmup}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step_ref["i"] = i
        for op in ops:
            op.fn()
    torch.cuda.synchronize()

    def timed_passes(sel):
        """`steps` passes over the ops in `sel`, each op between its own event
        pair; returns the wall time per pass in ms."""
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sel]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for st in range(args.steps):
            step_ref["i"] = args.warmup + st
            for j, op in enumerate(sel):
                evs[st][j][0].record(stream)
                op.fn()
                evs[st][j][1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for st in range(args.steps):
            for j, op in enumerate(sel):
                op.times_ms.append(evs[st][j][0].elapsed_time(evs[st][j][1]))
        return (t1 - t0) * 1e3 / args.steps

    step_ops = [op for op in ops if op.in_step]
    extra_ops = [op for op in ops if not op.in_step]
    ms_per_step = timed_passes(step_ops) if step_ops else 0.0
    print(f"bench: timed {args.steps} steps, {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    if extra_ops:
        timed_passes(extra_ops)
        print(f"bench: timed {len(extra_ops)} further ops outside the step", file=sys.stderr, flush=True)

    # Back-to-back launches: R launches of the op (decode ops on R successive
    # weight copies) captured once into a HIP graph, so that the host's
    # per-call Python and launch overhead stays out of the GPU timeline, and
    # the graph replayed `steps` times, one event pair per replay.
    launch = args.warmup + args.steps
    for op in ops:
        op.reps = int(min(64, max(1, round(1.0 / max(float(np.median(op.times_ms)), 1e-3)))))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(op.reps):
                step_ref["i"] = launch
                launch += 1
                op.fn()
        graph.replay()
        torch.cuda.synchronize()
        # at least 7 replays and 200 launches per op
        replays = max(args.steps, 7, -(-200 // op.reps))
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(replays)]
        for e0, e1 in pairs:
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        op.batch_ms = [e0.elapsed_time(e1) / op.reps for e0, e1 in pairs]
        del graph
    print("bench: timed back-to-back launches (graph replays)", file=sys.stderr, flush=True)
    copy_gbs = measured_copy_gbs(torch, dev, stream, args.steps)

    kernels = []
    for op in ops:
        t = np.array(op.batch_ms)
        ms = float(np.mean(t))
        rl = op.roofline(ms)
        entry = {"op": op.name, "format": op.fmt, "kind": op.kind, "in_step": op.in_step, "ms": ms,
                 "ms_median": float(np.median(t)),
                 "cv": float(np.std(t) / ms) if ms > 0 else 0.0, "reps": op.reps, "launches": op.reps * len(t),
                 "ms_in_step": float(np.mean(op.times_ms)), "bytes": op.nbytes, "flops": op.flops, **rl}
        if op.kind in ("prefill", "sweep") and op.peak_key in ("f16", "bf6"):
            entry["frac_int8_peak"] = rl["achieved"] / PEAK_TFLOPS["i8"]
        if op.kind == "prefill" and op.peak_key == "bf6":
            entry["frac_f16_peak"] = rl["achieved"] / PEAK_TFLOPS["f16"]
        if op.name == "ternary_gemm":
            entry["hbm_gbs"] = op.nbytes / (ms * 1e-3) / 1e9
            entry["hbm_frac"] = entry["hbm_gbs"] / PEAK_HBM_GBS
        if rl["bound"] == "hbm" and copy_gbs:
            entry["frac_of_copy"] = rl["achieved"] / copy_gbs
        entry["noisy"] = entry["cv"] > NOISY_CV
        kernels.append(entry)
        print(f"  {op.name:22s} {ms * 1e3:10.2f} us (in step {entry['ms_in_step'] * 1e3:8.2f})  "
              f"{rl['achieved']:10.1f} {rl['unit']:8s} "
              f"{100 * rl['frac']:6.1f}% of {rl['bound']} peak  (cv {entry['cv']:.3f})", file=sys.stderr)
    # the whole per-kernel table, on stderr (and in a file when asked), so
    # that stdout ends with one short line
    table = json.dumps({"kernels": kernels})
    print("bench kernels: " + table, file=sys.stderr, flush=True)
    if args.kernels_out:
        with open(args.kernels_out, "w") as f:
            f.write(table + "\n")

    def agg(fmt, kind):
        sel = [(op, e) for op, e in zip(ops, kernels) if op.fmt == fmt and op.kind == kind]
        if not sel:
            return None
        t = sum(e["ms"] for _, e in sel) * 1e-3
        if kind == "decode":
            v = sum(op.nbytes for op, _ in sel) / t / 1e9
            return {"gbs": r4(v), "frac": r4(v / PEAK_HBM_GBS)}
        v = sum(op.flops for op, _ in sel) / t / 1e12
        key = sel[0][0].peak_key
        out = {"tops": r4(v), "peak": key, "frac": r4(v / PEAK_TFLOPS[key])}
        if key in ("f16", "bf6"):
            out["frac_i8"] = r4(v / PEAK_TFLOPS["i8"])
        if key == "bf6":
            out["frac_f16"] = r4(v / PEAK_TFLOPS["f16"])
        return out

    per_format = {}
    for fmt in ("q4_0", "q4_0_repacked", "q4_0_decode_packed", "q8_0", "f32", "f32_core", "f32_nt", "bf16_nt",
                "f16_nt", "ternary"):
        d = {kind: agg(fmt, kind) for kind in ("decode", "prefill")}
        d = {kind: v for kind, v in d.items() if v}
        if d:
            per_format[fmt] = d

    by_name = {e["op"]: e for e in kernels}
    in_step = [e for e in kernels if e["in_step"]] or kernels
    dom = max(in_step, key=lambda e: e["ms"]) if in_step else None
    roofline = None
    if dom is not None:
        roofline = {"kernel": dom["op"], "bound": dom["bound"], "achieved": r4(dom["achieved"]), "peak": dom["peak"],
                    "unit": dom["unit"], "frac": r4(dom["frac"]), "traffic": traffic_for(dom["op"]),
                    "algorithmic_per_launch": dom["bytes"] if dom["bound"] == "hbm" else dom["flops"],
                    "algorithmic_unit": "bytes" if dom["bound"] == "hbm" else "flop",
                    "us_per_launch": r4(dom["ms"] * 1e3), "launches_timed": dom["launches"]}

    def us(name):
        e = by_name.get(name)
        return r4(e["ms"] * 1e3) if e else None

    rows = {
        "q4_gemv_512x512_us": us("q4_gemv_small"),
        "q4_decode_us": [us(f"q4_gemv_{s}") for s in range(4)],
        "q4_prefill_us": [us(f"q4_gemm_{s}") for s in range(4)],
        "q4_prefill_repacked_us": [us(f"q4r_gemm_{s}") for s in range(4)],
        "q4_decode_packed_us": [us(f"q4p_gemv_{s}") for s in range(4)],
        "sgemm_4096_us": us("sgemm_4096"), "sgemv_4096_us": us("sgemv_4096"),
        "ternary_m1_us": us("ternary_gemv"), "ternary_m64_us": us("ternary_gemm"),
        "m_sweep_4096x14336_us": {str(m): us(f"msweep_q4_m{m}") for m in M_SWEEP if f"msweep_q4_m{m}" in by_name},
        "fused_vs_pair_us": {f"m{m}": [[us(f"f1_fused_m{m}_{s}"), us(f"f1_pair_m{m}_{s}")] for s in range(4)]
                             for m in (1, 8)},
        "noisy": [e["op"] for e in kernels if e["noisy"]],
    }

    value = per_format.get("q4_0", {}).get("decode", {}) or {}
    cpu = None
    if not args.no_cpu_baseline and not args.only:
        print("bench: timing the oracle on the host (cpu_baseline)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(synth, np, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": r4(value.get("gbs")), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r4(ms_per_step), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": "one pass of the path: Q4_0 x Q8_0 GEMV 512x512; decode GEMV (m=1) and prefill GEMM "
                               "(m=512) on (k,n) = (4096,14336), (14336,4096), (4096,4096), (4096,128256) with their "
                               "Q8_0 quantization; f32 GEMM 4096^3 and GEMV 4096^2; BitNet ternary 2560->6912 at "
                               "m=1 and m=64 with int8 quantization",
                   "value_is": "Q4_0 x Q8_0 decode GEMV algorithmic bytes / summed average launch time over "
                               "the four 8B-class shapes (weights rotating through >= 1 GiB of copies)",
                   "parallelism": "single GPU"},
        "roofline": roofline, "per_format": per_format, "rows": rows, "cpu_baseline": cpu,
        "device": device_record(torch, dev, copy_gbs),
    }
    print(json.dumps(line, separators=(",", ":")), flush=True)


def r4(v):
    """Four significant digits (keeps the result line short)."""
    return None if v is None else float(f"{v:.4g}")


def measured_copy_gbs(torch, dev, stream, reps):
    """Secondary HBM denominator: a plain 1 GiB device-to-device copy (read +
    write bytes over its time), median of `reps` event-timed copies."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(max(3, reps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    t = sorted(ts)[len(ts) // 2]
    return 2 * (1 << 30) / (t * 1e-3) / 1e9


def device_record(torch, dev, copy_gbs):
    import glob
    import hashlib
    p = torch.cuda.get_device_properties(dev)
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "quantized_linear_layer_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "hip": torch.version.hip, "copy_1gib_gbs": r4(copy_gbs), "sclk_mhz": sclk_mhz(),
            "csrc_sha256_16": h.hexdigest()[:16], "date_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}


def sclk_mhz():
    """The GPU's current shader clock as amd-smi reports it (None if unavailable).

    amd-smi is a Python script; it is run as a child of this interpreter
    binary directly, so that no launcher (a `#!/usr/bin/env` hop) replaces
    itself by exec in a process that may already hold the GPU.  Under a
    profiler, whose preloaded library initialises the GPU in every child,
    the clock is not read at all."""
    import re
    import shutil
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return None
    tool = shutil.which("amd-smi")
    if tool is None:
        return None
    try:
        r = subprocess.run([sys.executable, tool, "metric", "-c", "-g", "0"], capture_output=True, text=True,
                           timeout=20)
    except (OSError, subprocess.TimeoutExpired):
        return None
    m = re.search(r"GFX_0:.*?CLK:\s*([0-9]+)\s*MHz", r.stdout, re.S)
    return int(m.group(1)) if m else None


def traffic_for(op_name):
    """HBM bytes per launch measured with rocprofv3 counters, read from the
    committed summary if it was taken on the current kernel sources."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    entry = rec.get("ops", {}).get(op_name)
    if not entry:
        return None
    src = os.path.join(ROOT, "quantized_linear_layer_amd", "csrc", entry["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != entry["source_sha256"]:
        return None
    return entry["bytes_per_launch"]


if __name__ == "__main__":
    main()
