"""GPU layer calls at the method's degenerate sizes and routings:
- no tokens (indexed, the entry point that allocates nothing, contiguous);
- top-1 routing;
- a single expert holding every row, on both schedules (one 128-row block
  or several);
- a token routed to the same expert in two of its top-k slots;
- a masked call whose every count is zero.

Each result is compared with the CPU oracle where there is one; the calls
without a result must succeed and leave the memory past their output
untouched.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare, require_gpu
from tests.test_gpu_a_kernels import tiny_weights
from tests.test_gpu_f_guards import canary_intact, guarded

pytestmark = pytest.mark.gpu


def test_no_tokens():
    require_gpu()
    import torch
    E, H, I, topk = 8, 256, 128, 2
    w = tiny_weights(E, H, I, seed=3)
    h = prepare(w, "indexed")
    x = torch.zeros((0, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((0, topk), dtype=torch.int32, device="cuda")
    tw = torch.zeros((0, topk), dtype=torch.float32, device="cuda")
    owhole, out = guarded(0, H)
    h.indexed(x, ids, tw, out=out)
    h.indexed_noalloc(x, ids, tw, out)
    torch.cuda.synchronize()
    assert canary_intact(owhole), "a call without tokens wrote to memory"
    hc = prepare(w, "contiguous")
    a = torch.zeros((0, H), dtype=torch.bfloat16, device="cuda")
    m_idx = torch.zeros((0,), dtype=torch.int32, device="cuda")
    owhole, out = guarded(0, H)
    hc.contiguous(a, m_idx, out=out)
    torch.cuda.synchronize()
    assert canary_intact(owhole), "a contiguous call without rows wrote to memory"


def test_top1_routing():
    require_gpu()
    E, H, I, T = 8, 256, 128, 61
    w = tiny_weights(E, H, I, seed=17)
    x = synth.activations(18, T, H)
    ids, tw = synth.softmax_routing(19, T, E, 1)
    h = prepare(w, "indexed")
    out = h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))
    check_tol(O.bf16_to_f64(bits_host(out)), O.moe_indexed(x, ids, tw, w, E=E), "top-1")


@pytest.mark.parametrize("T,schedule", [(20, "small-M"), (150, "large-M")])
def test_single_expert(T, schedule):
    """E = 1, top-1: every token on expert 0. 150 rows take large-M with two
    128-row blocks (one of 22 rows); 20 rows take small-M."""
    require_gpu()
    E, H, I = 1, 256, 256
    log(f"case single expert T={T} ({schedule})")
    w = tiny_weights(E, H, I, seed=23 + T)
    x = synth.activations(24, T, H)
    ids = np.zeros((T, 1), np.int32)
    tw = synth.rng(25, T).uniform(0.05, 1.0, size=(T, 1)).astype(np.float32)
    h = prepare(w, "indexed")
    assert f"schedule={schedule}" in h.describe(T, 1)
    out = h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))
    check_tol(O.bf16_to_f64(bits_host(out)), O.moe_indexed(x, ids, tw, w, E=E), "single expert")


def test_repeated_expert_in_a_token():
    """Rows are independent: a token whose top-k names one expert twice gets
    both weighted rows, as the oracle sums them."""
    require_gpu()
    E, H, I, T, topk = 8, 256, 128, 40, 4
    w = tiny_weights(E, H, I, seed=29)
    x = synth.activations(30, T, H)
    ids, tw = synth.softmax_routing(31, T, E, topk)
    ids[::3, 1] = ids[::3, 0]   # every third token: slots 0 and 1 on one expert
    h = prepare(w, "indexed")
    out = h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))
    check_tol(O.bf16_to_f64(bits_host(out)), O.moe_indexed(x, ids, tw, w, E=E), "repeated expert")


def test_masked_all_counts_zero():
    """Every expert's masked_m is 0: no row is valid, so the output holds
    nothing specified; the call must succeed and stay inside it."""
    require_gpu()
    import torch
    E, H, I, max_m = 6, 256, 128, 32
    w = tiny_weights(E, H, I, seed=37)
    a3 = synth.activations(38, E * max_m, H).reshape(E, max_m, H)
    h = prepare(w, "masked")
    owhole, out = guarded(E * max_m, H)
    for em in (1, 16, 200):
        h.masked(bf16_dev(a3), i32_dev(np.zeros(E, np.int32)), em, out=out)
    torch.cuda.synchronize()
    assert canary_intact(owhole), "the layer wrote past its output"
