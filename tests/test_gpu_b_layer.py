"""GPU parity of the whole layer against the CPU oracle, at sizes the oracle
finishes in seconds: every layout, several tiles, ragged row counts, K
tails, overrides, NaN-poisoned padding. Tolerance: relative Frobenius error
<= 5e-3 and max-abs error <= 3e-2 * rms(ref) against the unrounded oracle;
the intermediate `a` is compared too (mismatches must be rare 1-ulp flips).
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import (a_mismatch, bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log,
                            prepare, require_gpu)
from tests.test_gpu_a_kernels import tiny_weights

pytestmark = pytest.mark.gpu


INDEXED_CASES = [
    # (E, H, I, T, topk, ovr)
    (8, 256, 512, 32, 2, None),            # config 0 shape
    (16, 160, 96, 37, 4, None),            # K tails: H = 128 + 32, I = 96 < 128; 3 row groups
    (32, 512, 256, 200, 8, None),          # ~50 rows/expert: four token tiles per pass
    (12, 256, 128, 300, 6, None),          # ~150 rows/expert: several passes per expert
    (16, 256, 128, 64, 4, {"block_m": 64}),
    (16, 256, 128, 64, 4, {"block_m": 128, "schedule": 1}),
    (384, 128, 64, 448, 8, None),          # config 1 routing shape, small weights
    (1024, 128, 64, 40, 8, None),          # 320 rows over 1024 experts: grid over the active ones
    (4096, 128, 64, 100, 8, None),         # the largest expert count a handle accepts
    (96, 128, 64, 24, 64, None),           # the largest top-k (64)
]


@pytest.mark.parametrize("E,H,I,T,topk,ovr", INDEXED_CASES)
def test_indexed_small(E, H, I, T, topk, ovr):
    require_gpu()
    log(f"case indexed E={E} H={H} I={I} T={T} topk={topk} ovr={ovr}")
    w = tiny_weights(E, H, I, seed=E + H)
    x = synth.activations(11, T, H)
    ids, tw = synth.softmax_routing(12, T, E, topk)
    h = prepare(w, "indexed")
    ids_d = i32_dev(ids)
    routing = h.align(ids_d, ovr=ovr)
    ws = None
    import torch
    ws = torch.empty(h.workspace_bytes(T, topk, T, ovr=ovr), dtype=torch.uint8, device="cuda")
    out = h.indexed(bf16_dev(x), ids_d, f32_dev(tw), routing=routing, ws=ws, ovr=ovr)
    torch.cuda.synchronize()
    ref, inter = O.moe_indexed(x, ids, tw, w, E=E, keep=True)
    check_tol(O.bf16_to_f64(bits_host(out)), ref, "indexed")
    # intermediate a: workspace rows at the routing's sorted slots
    lay = h.routing_layout(T, topk, ovr)
    r = routing.cpu().numpy()
    sid = r[lay.off_sorted:lay.off_sorted + lay.cap]
    a_ws = ws[: lay.cap * I * 2].view(torch.int16).view(lay.cap, I).cpu().numpy().view(np.uint16)
    slots = np.flatnonzero(sid < T * topk)
    got_a = a_ws[slots]
    ref_a = np.stack([inter["a"][int(f)] for f in sid[slots]])
    frac, mx, within = a_mismatch(got_a, ref_a, "indexed")
    assert within and frac < 1e-3


def test_indexed_internal_routing_matches_explicit():
    require_gpu()
    E, H, I, T, topk = 16, 256, 128, 77, 4
    w = tiny_weights(E, H, I, seed=5)
    x = bf16_dev(synth.activations(1, T, H))
    ids, tw = synth.softmax_routing(2, T, E, topk)
    h = prepare(w, "indexed")
    out1 = h.indexed(x, i32_dev(ids), f32_dev(tw))
    out2 = h.indexed(x, i32_dev(ids), f32_dev(tw), routing=h.align(i32_dev(ids)))
    ref = O.moe_indexed(synth.activations(1, T, H), ids, tw, w, E=E)
    check_tol(O.bf16_to_f64(bits_host(out1)), ref, "internal routing")
    check_tol(O.bf16_to_f64(bits_host(out2)), ref, "explicit routing")


def test_indexed_dropped_ids_and_unrouted_tokens():
    """Ids outside [0, E) route nowhere; a token with no valid id gets 0."""
    require_gpu()
    E, H, I, T, topk = 8, 256, 128, 40, 3
    w = tiny_weights(E, H, I, seed=8)
    x = synth.activations(3, T, H)
    ids, tw = synth.softmax_routing(4, T, E, topk)
    ids[::5, 1] = -1
    ids[7, :] = -1
    ids[9, 2] = E + 3
    h = prepare(w, "indexed")
    out = O.bf16_to_f64(bits_host(h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))))
    ref = O.moe_indexed(x, ids, tw, w, E=E)
    assert np.all(out[7] == 0)
    check_tol(out, ref, "dropped ids")


def test_routing_made_for_other_shapes_is_ignored():
    """A routing aligned with another block size computes nothing (no fault)."""
    require_gpu()
    E, H, I, T, topk = 8, 256, 128, 40, 2
    w = tiny_weights(E, H, I, seed=9)
    x = bf16_dev(synth.activations(3, T, H))
    ids, tw = synth.softmax_routing(4, T, E, topk)
    h = prepare(w, "indexed")
    routing = h.align(i32_dev(ids), ovr={"block_m": 64})
    out = h.indexed(x, i32_dev(ids), f32_dev(tw), routing=routing, ovr={"block_m": 128})
    assert np.all(bits_host(out) == 0)


MASKED_CASES = [
    # (E, H, I, max_m, expected_m)
    (8, 256, 128, 40, 16),
    (6, 160, 96, 64, 16),
    (5, 256, 128, 100, 50),
    (4, 256, 128, 7, 1),
]


@pytest.mark.parametrize("E,H,I,max_m,expected_m", MASKED_CASES)
def test_masked_small(E, H, I, max_m, expected_m):
    require_gpu()
    log(f"case masked E={E} H={H} I={I} max_m={max_m} expected_m={expected_m}")
    w = tiny_weights(E, H, I, seed=E * 7 + max_m)
    a3 = synth.activations(21, E * max_m, H).reshape(E, max_m, H)
    mm = synth.rng(22, 14).integers(0, max_m + 1, size=E).astype(np.int32)
    mm[0], mm[-1] = 0, max_m
    a3p = a3.copy()
    for e in range(E):
        a3p[e, mm[e]:] = 0x7FC0           # rows beyond masked_m are NaN: must not leak
    h = prepare(w, "masked")
    out = O.bf16_to_f64(bits_host(h.masked(bf16_dev(a3p), i32_dev(mm), expected_m)))
    ref = O.moe_masked(a3, mm, w)
    valid = np.concatenate([np.arange(e * max_m, e * max_m + mm[e]) for e in range(E)])
    check_tol(out[valid], ref[valid], "masked")


def test_masked_expected_m_only_picks_the_launch():
    require_gpu()
    E, H, I, max_m = 6, 256, 128, 48
    w = tiny_weights(E, H, I, seed=31)
    a3 = synth.activations(5, E * max_m, H).reshape(E, max_m, H)
    mm = np.array([0, 48, 17, 1, 33, 16], dtype=np.int32)
    h = prepare(w, "masked")
    ref = O.moe_masked(a3, mm, w)
    valid = np.concatenate([np.arange(e * max_m, e * max_m + mm[e]) for e in range(E)])
    for em in (1, 16, 64, 200):
        out = O.bf16_to_f64(bits_host(h.masked(bf16_dev(a3), i32_dev(mm), em)))
        check_tol(out[valid], ref[valid], f"masked expected_m={em}")


CONTIG_CASES = [
    # (E, H, I, T, topk, extra_pad_blocks, with_row_src)
    (8, 256, 128, 100, 4, 0, True),
    (8, 256, 128, 100, 4, 2, True),
    (12, 160, 96, 150, 3, 1, False),
    (12, 160, 96, 150, 3, 1, True),        # H = 160: weighted rows padded to 192 features
    (4, 256, 128, 300, 2, 0, True),        # several 128-row blocks per expert
]


@pytest.mark.parametrize("E,H,I,T,topk,extra,with_src", CONTIG_CASES)
def test_contiguous_small(E, H, I, T, topk, extra, with_src):
    require_gpu()
    log(f"case contiguous E={E} H={H} I={I} T={T} topk={topk} extra={extra} row_src={with_src}")
    w = tiny_weights(E, H, I, seed=E + T)
    x = synth.activations(31, T, H)
    ids, tw = synth.softmax_routing(32, T, E, topk)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128, rows=a.shape[0] + 128 * extra)
    a_nan = a.copy()
    a_nan[m_idx < 0] = 0x7FC0             # pad rows are NaN: must not leak
    h = prepare(w, "contiguous")
    if with_src:
        out = h.contiguous(bf16_dev(a_nan), i32_dev(m_idx), i32_dev(row_src), f32_dev(tw), T, topk)
        ref = O.moe_contiguous(a, m_idx, w, row_src=row_src, topk_w=tw, T=T, topk=topk)
        check_tol(O.bf16_to_f64(bits_host(out)), ref, "contiguous+combine")
    else:
        out = h.contiguous(bf16_dev(a_nan), i32_dev(m_idx))
        ref = O.moe_contiguous(a, m_idx, w)
        valid = m_idx >= 0
        check_tol(O.bf16_to_f64(bits_host(out))[valid], ref[valid], "contiguous rows")


def test_layouts_agree_on_identical_routing():
    """The same routing through indexed, contiguous and masked gives the same
    per-row results within the tolerance (each against the oracle) and, for
    indexed vs contiguous+combine, close outputs."""
    require_gpu()
    E, H, I, T, topk = 8, 256, 128, 60, 2
    w = tiny_weights(E, H, I, seed=77)
    x = synth.activations(41, T, H)
    ids, tw = synth.softmax_routing(42, T, E, topk)
    ref = O.moe_indexed(x, ids, tw, w, E=E)
    hi, hc = prepare(w, "indexed"), prepare(w, "contiguous")
    out_i = O.bf16_to_f64(bits_host(hi.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))))
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    out_c = O.bf16_to_f64(bits_host(hc.contiguous(bf16_dev(a), i32_dev(m_idx), i32_dev(row_src),
                                                  f32_dev(tw), T, topk)))
    check_tol(out_i, ref, "indexed")
    check_tol(out_c, ref, "contiguous")
    check_tol(out_c, out_i, "contiguous vs indexed")


DISPATCH_CASES = [
    # (E, H, I, T, topk, grid cap or 0): the persistent small-M forms on
    # routing blocks of one weight pass; capped grids make every workgroup
    # walk many jobs across blocks. K chunks 1 (H 128, I 64 with a K tail),
    # 2 (256) and 3 (384); one, two and four token tiles per pass.
    (16, 128, 64, 40, 4, 0),
    (16, 128, 64, 40, 4, 1),
    (16, 256, 256, 100, 4, 3),
    (8, 384, 384, 60, 4, 5),
    (12, 256, 128, 120, 6, 2),
    (384, 128, 64, 448, 8, 0),
]


@pytest.mark.parametrize("dispatch", [1, 2, 3])
@pytest.mark.parametrize("E,H,I,T,topk,wgs", DISPATCH_CASES)
def test_indexed_small_dispatch(E, H, I, T, topk, wgs, dispatch, monkeypatch):
    """Persistent static and job-queue dispatch, and the semi-static grid over
    routing blocks, against the oracle: outputs and the intermediate a, with
    the persistent forms' weight and token streams running on across job
    boundaries."""
    require_gpu()
    import torch
    log(f"case dispatch={dispatch} E={E} H={H} I={I} T={T} topk={topk} wgs={wgs}")
    if wgs:
        monkeypatch.setenv("MOE_W4A16_JOB_WGS", str(wgs))
    ovr = {"dispatch": dispatch}
    w = tiny_weights(E, H, I, seed=E * 3 + I)
    x = synth.activations(41, T, H)
    ids, tw = synth.zipf_routing(42, T, E, topk)
    ids = ids.copy()
    ids[::7, 0] = -1
    h = prepare(w, "indexed")
    d = h.describe(T, topk, ovr=ovr)
    log(f"  {d}")
    assert "small-M" in d and ("dispatch=persistent" in d if dispatch < 3 else "semi-static-blocks" in d)
    ids_d = i32_dev(ids)
    routing = h.align(ids_d, ovr=ovr)
    ws = torch.empty(h.workspace_bytes(T, topk, T, ovr=ovr), dtype=torch.uint8, device="cuda")
    out = h.indexed(bf16_dev(x), ids_d, f32_dev(tw), routing=routing, ws=ws, ovr=ovr)
    torch.cuda.synchronize()
    ref, inter = O.moe_indexed(x, ids, tw, w, E=E, keep=True)
    check_tol(O.bf16_to_f64(bits_host(out)), ref, f"indexed dispatch {dispatch}")
    lay = h.routing_layout(T, topk, ovr)
    r = routing.cpu().numpy()
    sid = r[lay.off_sorted:lay.off_sorted + lay.cap]
    a_ws = ws[: lay.cap * I * 2].view(torch.int16).view(lay.cap, I).cpu().numpy().view(np.uint16)
    slots = np.flatnonzero(sid < T * topk)
    ref_a = np.stack([inter["a"][int(f)] for f in sid[slots]])
    frac, mx, within = a_mismatch(a_ws[slots], ref_a, f"indexed dispatch {dispatch}")
    assert within and frac < 1e-3
    # the same call again: the queue is cleared by each call
    out2 = h.indexed(bf16_dev(x), ids_d, f32_dev(tw), routing=routing, ws=ws, ovr=ovr)
    assert np.array_equal(bits_host(out2), bits_host(out))


@pytest.mark.parametrize("Eg,E,H,I,T,topk,placement", [
    (64, 8, 256, 128, 200, 8, "contiguous"),     # decode-like share: ~25 local rows per expert
    (64, 8, 256, 128, 200, 8, "round-robin"),
    (32, 4, 256, 256, 640, 4, "contiguous"),     # prefill-like share: ~80 rows per expert (large-M)
    (64, 8, 256, 128, 1, 4, "round-robin"),      # one token: fewer rows than local experts
])
def test_indexed_ep_share(Eg, E, H, I, T, topk, placement):
    """The layer on one GPU's expert share: only local rows are summed, tokens
    with no local expert get 0 (the partial output of an EP combine)."""
    require_gpu()
    from tests.test_gpu_a_kernels import ep_map
    log(f"case ep-share Eg={Eg} E={E} H={H} I={I} T={T} topk={topk} {placement}")
    w = tiny_weights(E, H, I, seed=Eg + E)
    x = synth.activations(51, T, H)
    ids, tw = synth.softmax_routing(52, T, Eg, topk)
    emap = ep_map(Eg, E, placement)
    ovr = {"global_experts": Eg}
    h = prepare(w, "indexed")
    log(f"  {h.describe(T, topk, ovr=ovr)}")
    routing = h.align_ep(i32_dev(ids), i32_dev(emap), Eg, ovr=ovr)
    out = O.bf16_to_f64(bits_host(h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw), routing=routing,
                                            ovr=ovr)))
    loc = O.ep_local_ids(ids, emap)
    ref = O.moe_indexed(x, loc, tw, w, E=E)
    none = np.all(loc < 0, axis=1)
    assert np.all(out[none] == 0)
    check_tol(out, ref, "indexed EP share")


SPLIT_CASES = [
    # (E, H, I, T, topk, forced split or 0 for the automatic choice, ovr):
    # grid-starved small-M calls split K over several workgroups and reduce
    # the partials (in split order) in the SwiGLU and in the combine
    (32, 2048, 1024, 1, 8, 0, None),        # one token: W13 split 2 (8 chunks each)
    (32, 2048, 1024, 3, 8, 0, None),
    (16, 384, 256, 40, 4, 2, None),         # forced: 3 chunks over 2 splits (uneven)
    (16, 160, 96, 37, 4, 2, None),          # forced: K tails, 2 chunks over 2 splits
    (16, 256, 128, 40, 4, 3, None),         # forced beyond the chunk count: capped
    (64, 1024, 512, 60, 8, 0, {"global_experts": 512}),   # an EP share's schedule
    (32, 2048, 1024, 1, 8, 1, None),        # forced 1: the active-expert grid (8 sets of 32) alone
    (32, 2048, 1024, 1, 8, 0, {"dispatch": 3}),           # over routing blocks
    (16, 384, 256, 40, 4, 2, {"dispatch": 3}),
]


@pytest.mark.parametrize("E,H,I,T,topk,split,ovr", SPLIT_CASES)
def test_indexed_small_split_k(E, H, I, T, topk, split, ovr, monkeypatch):
    require_gpu()
    import torch
    log(f"case split-K E={E} H={H} I={I} T={T} topk={topk} split={split} ovr={ovr}")
    if split:
        monkeypatch.setenv("MOE_W4A16_KSPLIT", str(split))
    w = tiny_weights(E, H, I, seed=E * 7 + H)
    x = synth.activations(61, T, H)
    ids, tw = synth.softmax_routing(62, T, E, topk)
    h = prepare(w, "indexed")
    d = h.describe(T, topk, ovr=ovr)
    log(f"  {d}")
    assert "small-M" in d
    if not split and not (ovr or {}).get("global_experts"):
        assert "ksplit=1/1" not in d
    ids_d = i32_dev(ids)
    routing = h.align(ids_d, ovr=ovr)
    ws = torch.empty(h.workspace_bytes(T, topk, T, ovr=ovr), dtype=torch.uint8, device="cuda")
    out = h.indexed(bf16_dev(x), ids_d, f32_dev(tw), routing=routing, ws=ws, ovr=ovr)
    torch.cuda.synchronize()
    ref, inter = O.moe_indexed(x, ids, tw, w, E=E, keep=True)
    check_tol(O.bf16_to_f64(bits_host(out)), ref, "indexed split-K")
    lay = h.routing_layout(T, topk, ovr)
    sid = routing.cpu().numpy()[lay.off_sorted:lay.off_sorted + lay.cap]
    a_ws = ws[: lay.cap * I * 2].view(torch.int16).view(lay.cap, I).cpu().numpy().view(np.uint16)
    slots = np.flatnonzero(sid < T * topk)
    ref_a = np.stack([inter["a"][int(f)] for f in sid[slots]])
    frac, mx, within = a_mismatch(a_ws[slots], ref_a, "indexed split-K")
    assert within and frac < 1e-3
    out2 = h.indexed(bf16_dev(x), ids_d, f32_dev(tw), routing=routing, ws=ws, ovr=ovr)
    assert np.array_equal(bits_host(out2), bits_host(out)), "split-K result depends on the run"
