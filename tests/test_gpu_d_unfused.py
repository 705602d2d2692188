"""GPU parity of the unfused steps of the indexed layer (gate_up GEMM with a
BF16 output, standalone SwiGLU, down GEMM with a BF16 output) against the
oracle's step functions, each fed the GPU's own input of that step, so every
comparison is of one step. BF16 outputs of FP32 accumulations may differ
from the float64 oracle by rare one-ulp flips near rounding boundaries:
the check is the one used for the fused path's intermediate `a`.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import a_mismatch, bf16_dev, bits_host, i32_dev, log, prepare, require_gpu
from tests.test_gpu_a_kernels import tiny_weights

pytestmark = pytest.mark.gpu

UNFUSED_CASES = [
    # (E, H, I, T, topk, routing, ovr)
    (16, 256, 128, 40, 4, "softmax", None),           # small-M, one token tile
    (16, 160, 96, 37, 4, "softmax", None),            # K tails, 3 row groups of W13
    (12, 256, 128, 120, 6, "softmax", None),          # small-M, four token tiles
    (8, 384, 256, 400, 4, "zipf", None),              # large-M (200 rows/expert), W2 K-resident
    (16, 256, 384, 300, 4, "zipf", {"schedule": 2}),  # forced large-M, K-loop W2 (3 chunks)
]


@pytest.mark.parametrize("E,H,I,T,topk,kind,ovr", UNFUSED_CASES)
def test_unfused_steps(E, H, I, T, topk, kind, ovr):
    require_gpu()
    import torch
    import w4a16_int4_grouped_amd as M
    log(f"case unfused E={E} H={H} I={I} T={T} topk={topk} {kind} ovr={ovr}")
    w = tiny_weights(E, H, I, seed=E * 13 + I)
    x = synth.activations(71, T, H)
    if kind == "zipf":
        ids, _ = synth.zipf_routing(72, T, E, topk)
    else:
        ids, _ = synth.softmax_routing(72, T, E, topk)
    ids = ids.copy()
    ids[::9, -1] = -1                                 # dropped rows leave pad slots
    h = prepare(w, "indexed")
    log(f"  {h.describe(T, topk, ovr=ovr)}")
    routing = h.align(i32_dev(ids), ovr=ovr)
    hout = h.gate_up(bf16_dev(x), topk, routing, ovr=ovr)
    a = M.swiglu(hout)
    y = h.down(a, T, topk, routing, ovr=ovr)
    torch.cuda.synchronize()
    lay = h.routing_layout(T, topk, ovr)
    sid = routing.cpu().numpy()[lay.off_sorted:lay.off_sorted + lay.cap]
    slots = np.flatnonzero(sid < T * topk)
    f = sid[slots].astype(np.int64)
    tok, ex = f // topk, ids.reshape(-1)[f]
    hg, ag, yg = bits_host(hout)[slots], bits_host(a)[slots], bits_host(y)[slots]
    ref_h = np.zeros_like(hg)
    ref_a = O.swiglu_rows(hg)
    ref_y = np.zeros_like(yg)
    for e in np.unique(ex):
        m = ex == e
        ref_h[m] = O.gate_up_rows(x[tok[m]], O.dequant(w[0][e], w[1][e]))
        ref_y[m] = O.down_rows(ag[m], O.dequant(w[2][e], w[3][e]))
    for what, got, ref in (("gate_up", hg, ref_h), ("swiglu", ag, ref_a), ("down", yg, ref_y)):
        frac, mx, within = a_mismatch(got, ref, what)
        assert within and frac < 1e-3, what


def test_swiglu_rejects_bad_shapes():
    require_gpu()
    import ctypes
    import torch
    import w4a16_int4_grouped_amd as M
    h = torch.zeros((4, 24), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda")
    st = M.lib().moe_swiglu(ctypes.c_void_p(h.data_ptr()), 4, 12, ctypes.c_void_p(a.data_ptr()), None)
    assert st == M.MOE_ERR_INVALID_ARG and "multiple of 8" in M.last_error()
