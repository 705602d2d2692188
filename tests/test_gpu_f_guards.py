"""Out-of-bounds guards for every entry point: each output buffer is followed
by canary bytes that must survive the call, and inputs are followed by a
NaN-poisoned guard row that must not reach any output (a kernel reading past
its input rows, e.g. through a pad sentinel T*topk used as a row index, would
turn outputs into NaN)."""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare, require_gpu
from tests.test_gpu_a_kernels import tiny_weights

pytestmark = pytest.mark.gpu

CANARY = 0x5A5A


def guarded(rows, cols, dtype="bf16"):
    """A device buffer of `rows` rows followed by one canary row; returns the
    (whole, view of the first rows) pair."""
    import torch
    tdt = {"bf16": torch.bfloat16, "i32": torch.int32, "f32": torch.float32}[dtype]
    whole = torch.empty((rows + 1, cols), dtype=tdt, device="cuda")
    whole.view(torch.int16).fill_(CANARY)
    return whole, whole[:rows]


def canary_intact(whole):
    import torch
    tail = whole[-1:].contiguous().view(torch.int16).cpu().numpy()
    return bool(np.all(tail == CANARY))


def with_nan_row(bits):
    """Device copy of a bf16 row-major array with one NaN row after it; returns
    the view of the real rows."""
    g = np.concatenate([bits, np.full((1,) + bits.shape[1:], synth.bf16_nan_bits(), np.uint16)])
    return bf16_dev(g)[: bits.shape[0]]


@pytest.mark.parametrize("E,H,I,T,topk,ovr", [
    (16, 256, 128, 37, 4, None),                 # small-M
    (16, 160, 96, 37, 4, None),                  # H = 160: weighted rows padded to 192 features
    (8, 256, 256, 400, 4, None),                 # large-M (200 rows / expert)
    (16, 256, 128, 37, 4, {"dispatch": 2}),      # persistent job queue
])
def test_indexed_guards(E, H, I, T, topk, ovr):
    require_gpu()
    import torch
    log(f"case indexed guards E={E} H={H} I={I} T={T} topk={topk} ovr={ovr}")
    w = tiny_weights(E, H, I, seed=E * 5 + T)
    x = synth.activations(111, T, H)
    ids, tw = synth.softmax_routing(112, T, E, topk)
    ids = ids.copy()
    ids[::6, -1] = -1
    h = prepare(w, "indexed")
    lay = h.routing_layout(T, topk, ovr)
    rwhole, routing = guarded(1, lay.total_ints, "i32")
    routing = routing.view(-1)
    h.align(i32_dev(ids), ovr=ovr, routing=routing)
    nws = h.workspace_bytes(T, topk, T, ovr=ovr)
    wwhole = torch.empty(nws + 256, dtype=torch.uint8, device="cuda")
    wwhole.view(torch.int16).fill_(CANARY)
    owhole, out = guarded(T, H)
    h.indexed(with_nan_row(x), i32_dev(ids), f32_dev(tw), routing=routing, out=out, ws=wwhole[:nws], ovr=ovr)
    torch.cuda.synchronize()
    assert canary_intact(rwhole), "align wrote past the routing buffer"
    assert canary_intact(owhole), "the layer wrote past its output"
    assert bool(torch.all(wwhole[nws:].view(torch.int16) == CANARY)), "the layer wrote past its workspace"
    check_tol(O.bf16_to_f64(bits_host(out)), O.moe_indexed(x, ids, tw, w, E=E), "indexed, guarded")
    # the unfused steps and the permute
    gwhole, gate_up = guarded(lay.cap, 2 * I)
    h.gate_up(with_nan_row(x), topk, routing, out=gate_up, ovr=ovr)
    import w4a16_int4_grouped_amd as M
    awhole, a = guarded(lay.cap, I)
    M.swiglu(gate_up, out=a)
    dwhole, down = guarded(lay.cap, H)
    h.down(a, T, topk, routing, out=down, ovr=ovr)
    torch.cuda.synchronize()
    for name, wh in (("gate_up", gwhole), ("swiglu", awhole), ("down", dwhole)):
        assert canary_intact(wh), f"{name} wrote past its output"
    sid = routing.cpu().numpy()[lay.off_sorted:lay.off_sorted + lay.cap]
    valid = sid < T * topk
    assert not np.any(np.isnan(O.bf16_to_f64(bits_host(down))[valid])), "a guard row reached the down rows"


def test_permute_guards():
    require_gpu()
    import torch
    E, H, T, topk = 12, 256, 50, 3
    h = prepare(tiny_weights(E, H, 64, seed=113), "indexed")
    x = synth.activations(114, T, H)
    ids, _ = synth.softmax_routing(115, T, E, topk)
    ovr = {"block_m": 128}
    routing = h.align(i32_dev(ids), ovr=ovr)
    lay = h.routing_layout(T, topk, ovr)
    import ctypes
    import w4a16_int4_grouped_amd as M
    awhole, a = guarded(lay.cap, H)
    mwhole, m = guarded(1, lay.cap, "i32")
    swhole, src = guarded(1, lay.cap, "i32")
    M.check(M.lib().moe_permute(h.handle, ctypes.c_void_p(with_nan_row(x).data_ptr()), T, topk, M._tuning(ovr),
                                ctypes.c_void_p(routing.data_ptr()), ctypes.c_void_p(a.data_ptr()),
                                ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(src.data_ptr()), None))
    torch.cuda.synchronize()
    for name, wh in (("a", awhole), ("m_indices", mwhole), ("row_src", swhole)):
        assert canary_intact(wh), f"permute wrote past {name}"
    ref_a, ref_m, ref_src = O.contiguous_layout(x, ids, E, 128)
    n = ref_a.shape[0]
    assert np.array_equal(bits_host(a)[:n], ref_a)
    assert np.array_equal(m.cpu().numpy().reshape(-1)[:n], ref_m)
    assert np.array_equal(src.cpu().numpy().reshape(-1)[:n], ref_src)
    # without a_out (x may then be NULL): only the two index arrays, the same
    m.fill_(7)
    src.fill_(7)
    M.check(M.lib().moe_permute(h.handle, None, T, topk, M._tuning(ovr), ctypes.c_void_p(routing.data_ptr()),
                                None, ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(src.data_ptr()), None))
    torch.cuda.synchronize()
    for name, wh in (("m_indices", mwhole), ("row_src", swhole)):
        assert canary_intact(wh), f"permute wrote past {name}"
    assert np.array_equal(m.cpu().numpy().reshape(-1)[:n], ref_m)
    assert np.array_equal(src.cpu().numpy().reshape(-1)[:n], ref_src)
    assert bool((m.reshape(-1)[n:] == -1).all()) and bool((src.reshape(-1)[n:] == -1).all())


@pytest.mark.parametrize("with_src", [True, False])
def test_contiguous_guards(with_src):
    require_gpu()
    import torch
    E, H, I, T, topk = 8, 256, 128, 90, 4
    w = tiny_weights(E, H, I, seed=116)
    x = synth.activations(117, T, H)
    ids, tw = synth.softmax_routing(118, T, E, topk)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    M_pad = a.shape[0]
    h = prepare(w, "contiguous")
    rows = T if with_src else M_pad
    owhole, out = guarded(rows, H)
    if with_src:
        h.contiguous(with_nan_row(a), i32_dev(m_idx), i32_dev(row_src), f32_dev(tw), T, topk, out=out)
        ref = O.moe_contiguous(a, m_idx, w, row_src=row_src, topk_w=tw, T=T, topk=topk)
        got = O.bf16_to_f64(bits_host(out))
    else:
        h.contiguous(with_nan_row(a), i32_dev(m_idx), out=out)
        keep = m_idx >= 0
        ref = O.moe_contiguous(a, m_idx, w)[keep]
        got = O.bf16_to_f64(bits_host(out))[keep]
    torch.cuda.synchronize()
    assert canary_intact(owhole), "the layer wrote past its output"
    check_tol(got, ref, "contiguous, guarded")


def test_masked_guards():
    require_gpu()
    import torch
    E, H, I, max_m = 6, 256, 128, 40
    w = tiny_weights(E, H, I, seed=119)
    a3 = synth.activations(120, E * max_m, H).reshape(E, max_m, H)
    mm = np.array([0, 40, 3, 17, 33, 1], np.int32)
    h = prepare(w, "masked")
    owhole, out = guarded(E * max_m, H)
    a3_d = with_nan_row(a3.reshape(E * max_m, H)).view(E, max_m, H)
    h.masked(a3_d, i32_dev(mm), 16, out=out)
    torch.cuda.synchronize()
    assert canary_intact(owhole), "the layer wrote past its output"
    got = O.bf16_to_f64(bits_host(out)).reshape(E, max_m, H)
    ref = O.moe_masked(a3, mm, w).reshape(E, max_m, H)
    valid = np.arange(max_m)[None, :] < mm[:, None]
    check_tol(got[valid], ref[valid], "masked, guarded")
