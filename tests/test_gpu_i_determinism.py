"""Run-to-run determinism of the layer: the same inputs give bit-identical
outputs on every call, whatever the stream, the buffers or the schedule.

No step accumulates through atomics: the alignment places rows by flat
index, each GEMM output element is written by one workgroup, split-K
partial sums are added in split order, and the combine sums a token's rows
in ascending j. The dynamic job queue (dispatch 2) changes which workgroup
computes a job, not how the job computes, so it is covered too. Each case
calls the layer three times: on a second stream with fresh output and
workspace, and again on the first stream into the first buffers.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare, require_gpu
from tests.test_gpu_a_kernels import tiny_weights

pytestmark = pytest.mark.gpu

INDEXED = [
    # (name, E, H, I, T, topk, routing, ovr)
    ("small-M semi-static", 64, 1024, 512, 200, 8, "softmax", None),
    ("small-M job queue", 64, 1024, 512, 200, 8, "softmax", {"dispatch": 2}),
    ("small-M split K (batch 1)", 64, 2048, 256, 1, 8, "softmax", None),
    ("large-M", 8, 512, 256, 600, 2, "zipf", None),
    ("large-M forced", 16, 512, 256, 160, 4, "softmax", {"schedule": 2}),
]


def _three_calls(call):
    """Outputs of call(stream, fresh) three times: default stream, a second
    stream with fresh buffers, the default stream again into the first."""
    import torch
    torch.cuda.synchronize()
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    first = call(s0, None)
    torch.cuda.synchronize()
    a = bits_host(first)
    with torch.cuda.stream(s1):
        b = bits_host_sync(call(s1, None))
    c = bits_host_sync(call(s0, first))
    return a, b, c


def bits_host_sync(t):
    import torch
    torch.cuda.synchronize()
    return bits_host(t)


@pytest.mark.parametrize("name,E,H,I,T,topk,routing,ovr", INDEXED, ids=[c[0] for c in INDEXED])
def test_indexed_is_deterministic(name, E, H, I, T, topk, routing, ovr):
    require_gpu()
    log(f"case determinism indexed {name}: E={E} H={H} I={I} T={T} topk={topk} ovr={ovr}")
    w = tiny_weights(E, H, I, seed=700 + E + T)
    h = prepare(w, "indexed")
    log(f"  {h.describe(T, topk, ovr=ovr)}")
    x = synth.activations(710 + T, T, H)
    route = synth.zipf_routing if routing == "zipf" else synth.softmax_routing
    ids, tw = route(720 + T, T, E, topk)
    x_d, ids_d, tw_d = bf16_dev(x), i32_dev(ids), f32_dev(tw)

    def call(stream, out):
        return h.indexed(x_d, ids_d, tw_d, out=out, ovr=ovr, stream=stream)

    a, b, c = _three_calls(call)
    assert np.any(a != 0), "all-zero output"
    assert np.array_equal(a, b), f"{name}: second stream differs"
    assert np.array_equal(a, c), f"{name}: repeated call differs"
    check_tol(O.bf16_to_f64(a), O.moe_indexed(x, ids, tw, w, E=E), f"determinism {name}")


def test_contiguous_is_deterministic():
    require_gpu()
    E, H, I, T, topk = 8, 512, 256, 400, 4
    log(f"case determinism contiguous + combine: E={E} H={H} I={I} T={T} topk={topk}")
    w = tiny_weights(E, H, I, seed=731)
    h = prepare(w, "contiguous")
    x = synth.activations(732, T, H)
    ids, tw = synth.zipf_routing(733, T, E, topk)
    a_np, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    log(f"  {h.describe(a_np.shape[0])}")
    a_d, m_d, s_d, tw_d = bf16_dev(a_np), i32_dev(m_idx), i32_dev(row_src), f32_dev(tw)

    def call(stream, out):
        return h.contiguous(a_d, m_d, s_d, tw_d, T, topk, out=out, stream=stream)

    a, b, c = _three_calls(call)
    assert np.any(a != 0)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    ref = O.moe_contiguous(a_np, m_idx, w, row_src=row_src, topk_w=tw, T=T, topk=topk)
    check_tol(O.bf16_to_f64(a), ref, "determinism contiguous")


def test_masked_is_deterministic():
    require_gpu()
    E, H, I, max_m, expected_m = 12, 768, 256, 64, 16
    log(f"case determinism masked: E={E} H={H} I={I} max_m={max_m} expected_m={expected_m}")
    w = tiny_weights(E, H, I, seed=741)
    h = prepare(w, "masked")
    log(f"  {h.describe(max_m, expected_m=expected_m)}")
    a3 = synth.activations(742, E * max_m, H).reshape(E, max_m, H)
    mm = synth.rng(743, 14).integers(0, max_m + 1, size=E).astype(np.int32)
    a3_d, mm_d = bf16_dev(a3), i32_dev(mm)

    def call(stream, out):
        return h.masked(a3_d, mm_d, expected_m, out=out, stream=stream)

    a, b, c = _three_calls(call)
    valid = np.concatenate([np.arange(e * max_m, e * max_m + mm[e]) for e in range(E)]).astype(np.int64)
    assert valid.size and np.any(a[valid] != 0)
    # rows past masked_m are unspecified; the valid rows must repeat exactly
    assert np.array_equal(a[valid], b[valid]) and np.array_equal(a[valid], c[valid])
    check_tol(O.bf16_to_f64(a)[valid], O.moe_masked(a3, mm, w)[valid], "determinism masked")
