"""Validation mode (MOE_W4A16_VALIDATE=1, read when weights are prepared):
index data that the kernels would silently drop, clamp or misread fails the
call on the host, and good data gives the same outputs as without the mode.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare, require_gpu
from tests.test_gpu_a_kernels import ep_map, tiny_weights

pytestmark = pytest.mark.gpu


@pytest.fixture
def validating(monkeypatch):
    monkeypatch.setenv("MOE_W4A16_VALIDATE", "1")


def expect_error(fn, status, text):
    import w4a16_int4_grouped_amd as M
    with pytest.raises(M.MoeError) as ei:
        fn()
    log(f"  rejected: {ei.value}")
    assert ei.value.status == status and text in str(ei.value)


def test_indexed_ids_and_routing(validating):
    require_gpu()
    import w4a16_int4_grouped_amd as M
    E, H, I, T, topk = 16, 256, 128, 50, 4
    w = tiny_weights(E, H, I, seed=91)
    x = bf16_dev(synth.activations(92, T, H))
    ids, tw = synth.softmax_routing(93, T, E, topk)
    ids = ids.copy()
    ids[::5, 1] = -1                              # -1 routes nowhere: accepted
    h = prepare(w, "indexed")
    out = h.indexed(x, i32_dev(ids), f32_dev(tw))
    check_tol(O.bf16_to_f64(bits_host(out)), O.moe_indexed(synth.activations(92, T, H), ids, tw, w, E=E),
              "validated indexed")
    bad = ids.copy()
    bad[7, 2] = E + 3
    expect_error(lambda: h.indexed(x, i32_dev(bad), f32_dev(tw)), M.MOE_ERR_INVALID_ARG, "topk_ids outside")
    bad[7, 2] = -2
    expect_error(lambda: h.align(i32_dev(bad)), M.MOE_ERR_INVALID_ARG, "topk_ids outside")
    # a routing made for another token count, and a buffer no alignment wrote
    other = h.align(i32_dev(ids[:T - 1]))
    expect_error(lambda: h.indexed(x, i32_dev(ids), f32_dev(tw), routing=other),
                 M.MOE_ERR_ROUTING_MISMATCH, "routing made for")
    import torch
    blank = torch.zeros_like(h.align(i32_dev(ids)))
    expect_error(lambda: h.indexed(x, i32_dev(ids), f32_dev(tw), routing=blank),
                 M.MOE_ERR_ROUTING_MISMATCH, "no alignment")
    expect_error(lambda: h.gate_up(x, topk, other), M.MOE_ERR_ROUTING_MISMATCH, "routing made for")
    # good routing through the unfused steps is accepted
    good = h.align(i32_dev(ids))
    M.swiglu(h.gate_up(x, topk, good))


def test_align_ep_map(validating):
    require_gpu()
    import w4a16_int4_grouped_amd as M
    Eg, E, T, topk = 64, 8, 40, 4
    h = prepare(tiny_weights(E, 128, 64, seed=94), "indexed")
    ids, _ = synth.softmax_routing(95, T, Eg, topk)
    emap = ep_map(Eg, E, "contiguous")
    h.align_ep(i32_dev(ids), i32_dev(emap), Eg)
    bad_map = emap.copy()
    bad_map[3] = E
    expect_error(lambda: h.align_ep(i32_dev(ids), i32_dev(bad_map), Eg), M.MOE_ERR_INVALID_ARG, "expert_map")
    bad_ids = ids.copy()
    bad_ids[0, 0] = Eg
    expect_error(lambda: h.align_ep(i32_dev(bad_ids), i32_dev(emap), Eg), M.MOE_ERR_INVALID_ARG,
                 "topk_ids outside")


def test_contiguous_blocks_and_row_src(validating):
    require_gpu()
    import w4a16_int4_grouped_amd as M
    E, H, I, T, topk = 8, 256, 128, 100, 4
    w = tiny_weights(E, H, I, seed=96)
    x = synth.activations(97, T, H)
    ids, tw = synth.softmax_routing(98, T, E, topk)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    h = prepare(w, "contiguous")
    ad, twd = bf16_dev(a), f32_dev(tw)
    out = h.contiguous(ad, i32_dev(m_idx), i32_dev(row_src), twd, T, topk)
    check_tol(O.bf16_to_f64(bits_host(out)),
              O.moe_contiguous(a, m_idx, w, row_src=row_src, topk_w=tw, T=T, topk=topk), "validated contiguous")
    rows = np.flatnonzero(m_idx >= 0)
    first = rows[0]
    assert rows[1] < 128                                 # the first block holds two rows
    cases = []
    m = m_idx.copy(); m[first] = E                       # expert id out of range
    cases.append((m, row_src, "m_indices outside"))
    m = m_idx.copy(); m[rows[1]] = (m[rows[1]] + 1) % E  # a second expert inside the first block
    cases.append((m, row_src, "two experts"))
    r = row_src.copy(); r[rows[1]] = r[rows[0]]          # one flat row feeding two rows
    cases.append((m_idx, r, "row_src"))
    pad = np.flatnonzero(m_idx < 0)
    r = row_src.copy(); r[pad[0]] = 0                    # a pad row with a source
    cases.append((m_idx, r, "row_src"))
    r = row_src.copy(); r[first] = T * topk              # source past the flat rows
    cases.append((m_idx, r, "row_src"))
    for m, r, text in cases:
        expect_error(lambda: h.contiguous(ad, i32_dev(m), i32_dev(r), twd, T, topk), M.MOE_ERR_INVALID_ARG, text)
    # without row_src only the experts are checked
    m = m_idx.copy(); m[rows[1]] = (m[rows[1]] + 1) % E
    expect_error(lambda: h.contiguous(ad, i32_dev(m)), M.MOE_ERR_INVALID_ARG, "two experts")


def test_masked_counts(validating):
    require_gpu()
    import w4a16_int4_grouped_amd as M
    E, H, I, max_m = 6, 256, 128, 32
    w = tiny_weights(E, H, I, seed=99)
    a3 = bf16_dev(synth.activations(100, E * max_m, H).reshape(E, max_m, H))
    mm = np.array([0, 5, 32, 17, 1, 9], np.int32)
    h = prepare(w, "masked")
    h.masked(a3, i32_dev(mm), 16)
    for v in (max_m + 1, -1):
        bad = mm.copy()
        bad[2] = v
        expect_error(lambda: h.masked(a3, i32_dev(bad), 16), M.MOE_ERR_INVALID_ARG, "masked_m")


def test_validated_outputs_match(monkeypatch):
    """The checks only read: a validated call's output is bit-identical to
    an unvalidated one's."""
    require_gpu()
    E, H, I, T, topk = 16, 256, 128, 64, 4
    w = tiny_weights(E, H, I, seed=101)
    x = bf16_dev(synth.activations(102, T, H))
    ids, tw = synth.softmax_routing(103, T, E, topk)
    plain = prepare(w, "indexed")
    monkeypatch.setenv("MOE_W4A16_VALIDATE", "1")
    checked = prepare(w, "indexed")
    a = bits_host(plain.indexed(x, i32_dev(ids), f32_dev(tw)))
    b = bits_host(checked.indexed(x, i32_dev(ids), f32_dev(tw)))
    assert np.array_equal(a, b)
