"""Graph capture of the layer. A layer call given its output and workspace
(or the no-allocation entry point) only launches kernels on the caller's
stream: no allocation, no synchronisation, no memset node (counters and
flags are cleared by fill kernels). A caller can therefore capture one call
into a HIP graph and replay it.

Each case warms the call up eagerly, captures it with its inputs in fixed
device buffers, then three times: writes new inputs into those buffers,
replays the graph, and compares the replay's output bit for bit with an
eager call on the same inputs into other buffers (eager work and
synchronisations between the replays, as a serving loop would have them).
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import bits_host, check_tol, log, prepare, require_gpu
from tests.test_gpu_a_kernels import tiny_weights

pytestmark = pytest.mark.gpu


def _to(t, arr):
    """Copy a host array into the device tensor t (same shape and width)."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    src = torch.from_numpy(a)
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).copy_(src)
    else:
        t.copy_(src)


def _replays(inputs_for, static, call, check_rows=None):
    """inputs_for(k): host arrays for replay k; static: device tensors they
    are copied into; call(out, stream) runs the layer on the static inputs."""
    import torch
    for t, a in zip(static, inputs_for(0)):
        _to(t, a)
    torch.cuda.synchronize()
    out_g = call(None, torch.cuda.current_stream())   # eager warmup; its buffers are the graph's
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g, torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs = []
    for k in range(3):
        for t, a in zip(static, inputs_for(k)):
            _to(t, a)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bits_host(out_g)
        ref = bits_host(call(None, torch.cuda.current_stream()))   # eager, fresh buffers
        torch.cuda.synchronize()
        rows = slice(None) if check_rows is None else check_rows(k)
        assert np.any(got[rows] != 0), f"replay {k}: all-zero output"
        assert np.array_equal(got[rows], ref[rows]), f"replay {k} differs from the eager call"
        outs.append(got)
    return outs


@pytest.mark.parametrize("name,E,H,I,T,topk,noalloc", [
    ("small-M", 64, 1024, 512, 200, 8, False),
    ("large-M", 8, 512, 256, 600, 2, False),
    ("no-allocation entry point", 32, 512, 256, 64, 4, True),
])
def test_indexed_graph(name, E, H, I, T, topk, noalloc):
    require_gpu()
    import torch
    log(f"case graph indexed {name}: E={E} H={H} I={I} T={T} topk={topk}")
    w = tiny_weights(E, H, I, seed=800 + E)
    h = prepare(w, "indexed")
    log(f"  {h.describe(T, topk)}")

    def inputs_for(k):
        x = synth.activations(810 + k, T, H)
        ids, tw = synth.softmax_routing(820 + k, T, E, topk) if k != 1 else synth.zipf_routing(820 + k, T, E, topk)
        return x, ids, tw

    x_s = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids_s = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    tw_s = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    ws = None if noalloc else torch.empty(h.workspace_bytes(T, topk, T), dtype=torch.uint8, device="cuda")

    def call(out, stream):
        # out None: an eager call into fresh buffers; else the captured call into out (and ws)
        if noalloc:
            if out is None:
                out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
            return h.indexed_noalloc(x_s, ids_s, tw_s, out, stream=stream)
        if out is None:
            return h.indexed(x_s, ids_s, tw_s, stream=stream)
        return h.indexed(x_s, ids_s, tw_s, out=out, ws=ws, stream=stream)

    outs = _replays(inputs_for, (x_s, ids_s, tw_s), call)
    x, ids, tw = inputs_for(2)
    check_tol(O.bf16_to_f64(outs[2]), O.moe_indexed(x, ids, tw, w, E=E), f"graph {name}, replay 2")


def test_contiguous_graph():
    require_gpu()
    import torch
    E, H, I, T, topk = 8, 512, 256, 300, 4
    log(f"case graph contiguous + combine: E={E} H={H} I={I} T={T} topk={topk}")
    w = tiny_weights(E, H, I, seed=831)
    h = prepare(w, "contiguous")
    routes = [synth.zipf_routing(840 + k, T, E, topk) for k in range(3)]
    xs = [synth.activations(850 + k, T, H) for k in range(3)]
    # one M_pad for every replay: the largest aligned total, as padding rows
    m_pad = max(O.align(r[0], E, 128)["total"] for r in routes)
    layouts = [O.contiguous_layout(xs[k], routes[k][0], E, 128, rows=m_pad) for k in range(3)]
    log(f"  {h.describe(m_pad)}")

    def inputs_for(k):
        a, m_idx, row_src = layouts[k]
        return a, m_idx, row_src, routes[k][1]

    a_s = torch.empty((m_pad, H), dtype=torch.bfloat16, device="cuda")
    m_s = torch.empty(m_pad, dtype=torch.int32, device="cuda")
    r_s = torch.empty(m_pad, dtype=torch.int32, device="cuda")
    tw_s = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(h.workspace_bytes(m_pad, topk, T), dtype=torch.uint8, device="cuda")

    def call(out, stream):
        if out is None:
            return h.contiguous(a_s, m_s, r_s, tw_s, T, topk, stream=stream)
        return h.contiguous(a_s, m_s, r_s, tw_s, T, topk, out=out, ws=ws, stream=stream)

    outs = _replays(inputs_for, (a_s, m_s, r_s, tw_s), call)
    a, m_idx, row_src = layouts[2]
    ref = O.moe_contiguous(a, m_idx, w, row_src=row_src, topk_w=routes[2][1], T=T, topk=topk)
    check_tol(O.bf16_to_f64(outs[2]), ref, "graph contiguous, replay 2")


def test_masked_graph():
    require_gpu()
    import torch
    E, H, I, max_m, expected_m = 12, 768, 256, 64, 16
    log(f"case graph masked: E={E} H={H} I={I} max_m={max_m} expected_m={expected_m}")
    w = tiny_weights(E, H, I, seed=861)
    h = prepare(w, "masked")
    log(f"  {h.describe(max_m, expected_m=expected_m)}")
    a3s = [synth.activations(870 + k, E * max_m, H).reshape(E, max_m, H) for k in range(3)]
    mms = [synth.rng(880 + k, 14).integers(0, max_m + 1, size=E).astype(np.int32) for k in range(3)]

    def inputs_for(k):
        return a3s[k], mms[k]

    def valid(k):
        return np.concatenate([np.arange(e * max_m, e * max_m + mms[k][e]) for e in range(E)]).astype(np.int64)

    a3_s = torch.empty((E, max_m, H), dtype=torch.bfloat16, device="cuda")
    mm_s = torch.empty(E, dtype=torch.int32, device="cuda")
    ws = torch.empty(h.workspace_bytes(max_m), dtype=torch.uint8, device="cuda")

    def call(out, stream):
        if out is None:
            return h.masked(a3_s, mm_s, expected_m, stream=stream)
        return h.masked(a3_s, mm_s, expected_m, out=out, ws=ws, stream=stream)

    outs = _replays(inputs_for, (a3_s, mm_s), call, check_rows=valid)
    v = valid(2)
    check_tol(O.bf16_to_f64(outs[2])[v], O.moe_masked(a3s[2], mms[2], w)[v], "graph masked, replay 2")
