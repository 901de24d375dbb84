"""The oracle's outputs at the workloads' full sizes, computed once per test
session and shared by the tests that check every output of a GPU path
against them (the direct and the repacked Q4_0 prefill GEMMs use the same
reference, as do the f32 GEMM on either matrix core).  Only oracle calls on
the seeded draws of synth.py; nothing here touches the GPU."""
import functools

import numpy as np

import oracle as O
import synth
from pins import np_pack_q8_0


@functools.lru_cache(maxsize=4)
def q4_prefill(s):
    """8B-class shape s at m = 512: (codes, d_bits, x, y_ref, mag), every output."""
    codes, d_bits, _ = synth.q4_decode(s)
    x = synth.q4_prefill_x(s)
    n, k = codes.shape
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), x.shape[0], n, k)
    return codes, d_bits, x, y_ref, mag


@functools.lru_cache(maxsize=1)
def q8w_prefill(s):
    """The same shape with Q8_0 weights: (block bytes from numpy, x, y_ref, mag)."""
    codes, d_bits, _ = synth.q8w_decode(s)
    x = synth.q4_prefill_x(s)
    n, k = codes.shape
    wq = np_pack_q8_0(codes, d_bits)
    y_ref, mag = O.q8_0_q8_0(wq, O.quantize_q8_0(x), x.shape[0], n, k)
    return wq, x, y_ref, mag


@functools.lru_cache(maxsize=1)
def sgemm_4096():
    """f32 GEMM 4096^3 of the workload: (a, b, c_ref, mag), every output."""
    a, b, _ = synth.f32_gemm()
    c_ref, mag = O.sgemm(a, b)
    return a, b, c_ref, mag


@functools.lru_cache(maxsize=2)
def gemm_nt_4096(wdtype):
    """Transposed-B GEMM 4096^3 with W = B^T of the f32 workload in `wdtype`
    (f32 as is; bf16 / f16 rounded to nearest even, as uint16 bits):
    (a, w, y_ref, mag), every output.  For f32 weights the definition is the
    plain GEMM's term for term, so its reference is sgemm_4096's."""
    if wdtype == "f32":
        a, b, c_ref, mag = sgemm_4096()
        return a, np.ascontiguousarray(b.T), c_ref, mag
    import torch
    a, b, _ = synth.f32_gemm()
    t = torch.from_numpy(np.ascontiguousarray(b.T)).to(torch.bfloat16 if wdtype == "bf16" else torch.float16)
    w = t.view(torch.int16).numpy().view(np.uint16).copy()
    y_ref, mag = O.gemm_nt(a, w, wdtype)
    return a, w, y_ref, mag
