"""GPU parity of the large-M schedule (128-row token tiles, token tile staged
through LDS) against the CPU oracle, at sizes the oracle finishes in
seconds: indexed routing blocks with skewed and empty experts, experts
spanning several blocks, odd and single K-chunk counts, dropped ids, the
contiguous layout with NaN padding, the masked layout with experts spanning
several tiles, and agreement with the small-M schedule on the same inputs.
Tolerance as for every layer output: relFro <= 5e-3, max-abs <= 3e-2 *
rms(ref).
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import (a_mismatch, bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log,
                            prepare, require_gpu)
from tests.test_gpu_a_kernels import tiny_weights

pytestmark = pytest.mark.gpu

LARGE = {"schedule": 2}


def describe(h, *a, **k):
    d = h.describe(*a, **k)
    log(f"  {d}")
    return d


LARGE_INDEXED = [
    # (E, H, I, T, topk, routing, ovr)
    (16, 256, 256, 400, 4, "zipf", None),      # ~100 rows/expert: auto large-M; skewed, some experts > 128
    (8, 384, 128, 340, 2, "softmax", None),    # 85 rows/expert; K chunks: 3 (odd) for W13, 1 for W2
    (24, 256, 128, 90, 4, "zipf", LARGE),      # forced large-M at 15 rows/expert: many empty experts
    (4, 128, 384, 700, 3, "softmax", LARGE),   # single W13 chunk; experts over 4 blocks
]


@pytest.mark.parametrize("E,H,I,T,topk,kind,ovr", LARGE_INDEXED)
def test_indexed_large(E, H, I, T, topk, kind, ovr):
    require_gpu()
    import torch
    log(f"case indexed-large E={E} H={H} I={I} T={T} topk={topk} {kind} ovr={ovr}")
    w = tiny_weights(E, H, I, seed=3 * E + H)
    x = synth.activations(51, T, H)
    if kind == "zipf":
        ids, tw = synth.zipf_routing(52, T, E, topk)
    else:
        ids, tw = synth.softmax_routing(52, T, E, topk)
    ids = ids.copy()
    ids[::11, -1] = -1                          # dropped rows
    h = prepare(w, "indexed")
    assert "schedule=large-M block=128" in describe(h, T, topk, ovr=ovr)
    ids_d = i32_dev(ids)
    routing = h.align(ids_d, ovr=ovr)
    ws = torch.empty(h.workspace_bytes(T, topk, T, ovr=ovr), dtype=torch.uint8, device="cuda")
    out = h.indexed(bf16_dev(x), ids_d, f32_dev(tw), routing=routing, ws=ws, ovr=ovr)
    torch.cuda.synchronize()
    ref, inter = O.moe_indexed(x, ids, tw, w, E=E, keep=True)
    check_tol(O.bf16_to_f64(bits_host(out)), ref, "indexed large-M")
    lay = h.routing_layout(T, topk, ovr)
    r = routing.cpu().numpy()
    sid = r[lay.off_sorted:lay.off_sorted + lay.cap]
    a_ws = ws[: lay.cap * I * 2].view(torch.int16).view(lay.cap, I).cpu().numpy().view(np.uint16)
    slots = np.flatnonzero(sid < T * topk)
    ref_a = np.stack([inter["a"][int(f)] for f in sid[slots]])
    frac, mx, within = a_mismatch(a_ws[slots], ref_a, "indexed large-M")
    assert within and frac < 1e-3


def test_large_and_small_schedules_agree():
    require_gpu()
    E, H, I, T, topk = 8, 256, 256, 200, 4
    w = tiny_weights(E, H, I, seed=99)
    x = synth.activations(61, T, H)
    ids, tw = synth.softmax_routing(62, T, E, topk)
    h = prepare(w, "indexed")
    ref = O.moe_indexed(x, ids, tw, w, E=E)
    outs = {}
    for sched in (1, 2):
        ovr = {"schedule": sched}
        describe(h, T, topk, ovr=ovr)
        outs[sched] = O.bf16_to_f64(bits_host(h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw), ovr=ovr)))
        check_tol(outs[sched], ref, f"schedule {sched}")
    check_tol(outs[2], outs[1], "large vs small")


def test_large_routing_made_for_other_block_is_ignored():
    require_gpu()
    E, H, I, T, topk = 8, 256, 128, 300, 2
    w = tiny_weights(E, H, I, seed=12)
    x = bf16_dev(synth.activations(3, T, H))
    ids, tw = synth.softmax_routing(4, T, E, topk)
    h = prepare(w, "indexed")
    routing = h.align(i32_dev(ids), ovr={"block_m": 64})
    out = h.indexed(x, i32_dev(ids), f32_dev(tw), routing=routing, ovr=LARGE)
    assert np.all(bits_host(out) == 0)


LARGE_CONTIG = [
    # (E, H, I, T, topk, extra_pad_blocks, with_row_src)
    (6, 384, 256, 250, 4, 1, True),
    (6, 384, 256, 250, 4, 0, False),
    (3, 256, 128, 500, 2, 2, True),             # experts over several blocks
]


@pytest.mark.parametrize("E,H,I,T,topk,extra,with_src", LARGE_CONTIG)
def test_contiguous_large(E, H, I, T, topk, extra, with_src):
    require_gpu()
    log(f"case contiguous-large E={E} H={H} I={I} T={T} topk={topk} extra={extra} row_src={with_src}")
    w = tiny_weights(E, H, I, seed=E * 5 + T)
    x = synth.activations(71, T, H)
    ids, tw = synth.zipf_routing(72, T, E, topk)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128, rows=a.shape[0] + 128 * extra)
    a_nan = a.copy()
    a_nan[m_idx < 0] = 0x7FC0
    h = prepare(w, "contiguous")
    assert "schedule=large-M" in describe(h, a.shape[0])
    if with_src:
        out = h.contiguous(bf16_dev(a_nan), i32_dev(m_idx), i32_dev(row_src), f32_dev(tw), T, topk)
        ref = O.moe_contiguous(a, m_idx, w, row_src=row_src, topk_w=tw, T=T, topk=topk)
        check_tol(O.bf16_to_f64(bits_host(out)), ref, "contiguous large-M + combine")
    else:
        out = h.contiguous(bf16_dev(a_nan), i32_dev(m_idx))
        ref = O.moe_contiguous(a, m_idx, w)
        valid = m_idx >= 0
        check_tol(O.bf16_to_f64(bits_host(out))[valid], ref[valid], "contiguous large-M rows")


@pytest.mark.parametrize("deal", ["0", "3", "16"])
def test_xcd_deal_settings(deal, monkeypatch):
    """The block -> workgroup mapping of the large-M K loop under other unit
    sizes: 0 (each XCD one contiguous range of blocks), 3 (units that do not
    divide the block count) and 16 (one unit larger than the routing). Indexed
    and contiguous, with an expert over several blocks."""
    require_gpu()
    monkeypatch.setenv("MOE_W4A16_XCD_DEAL", deal)
    E, H, I, T, topk = 5, 256, 128, 420, 2
    log(f"case xcd deal {deal}: E={E} H={H} I={I} T={T} topk={topk}")
    w = tiny_weights(E, H, I, seed=91)
    x = synth.activations(92, T, H)
    ids, tw = synth.zipf_routing(93, T, E, topk)
    hi = prepare(w, "indexed")
    assert "schedule=large-M" in hi.describe(T, topk)
    out = hi.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))
    check_tol(O.bf16_to_f64(bits_host(out)), O.moe_indexed(x, ids, tw, w, E=E), f"indexed deal {deal}")
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    hc = prepare(w, "contiguous")
    out = hc.contiguous(bf16_dev(a), i32_dev(m_idx), i32_dev(row_src), f32_dev(tw), T, topk)
    ref = O.moe_contiguous(a, m_idx, w, row_src=row_src, topk_w=tw, T=T, topk=topk)
    check_tol(O.bf16_to_f64(bits_host(out)), ref, f"contiguous deal {deal}")


def test_masked_large():
    """expected_m >= 80 picks large-M; experts of 0, 1, 129 and 300 valid rows
    (one, two and three tiles); rows past masked_m are NaN."""
    require_gpu()
    E, H, I, max_m = 4, 256, 128, 300
    w = tiny_weights(E, H, I, seed=41)
    a3 = synth.activations(81, E * max_m, H).reshape(E, max_m, H)
    mm = np.array([0, 1, 129, 300], dtype=np.int32)
    a3p = a3.copy()
    for e in range(E):
        a3p[e, mm[e]:] = 0x7FC0
    h = prepare(w, "masked")
    assert "schedule=large-M" in describe(h, max_m, expected_m=150)
    out = O.bf16_to_f64(bits_host(h.masked(bf16_dev(a3p), i32_dev(mm), 150)))
    ref = O.moe_masked(a3, mm, w)
    valid = np.concatenate([np.arange(e * max_m, e * max_m + mm[e]) for e in range(E)])
    check_tol(out[valid], ref[valid], "masked large-M")


MULTI_BLOCK_CASES = [
    # (E, H, I, T, topk, layout, with_row_src): K = 384 (3 chunks, an odd count)
    # on both GEMMs, hundreds of rows per expert spread over up to 6 blocks
    # with a Zipf skew, full and partial blocks side by side
    (6, 384, 384, 800, 3, "indexed", True),
    (5, 384, 384, 700, 2, "contiguous", True),
    (5, 384, 384, 700, 2, "contiguous", False),
]


WIDE_CASES = [
    # K = 512 on both GEMMs (4 chunks: whole chunk pairs) so that the 256-row
    # form runs both; Zipf-skewed experts give full same-expert block pairs,
    # pairs split between two experts and partial last blocks
    (6, 512, 512, 800, 3, "indexed", True),
    (5, 512, 512, 700, 2, "contiguous", True),
    (5, 512, 512, 700, 2, "contiguous", False),
]


@pytest.mark.parametrize("E,H,I,T,topk,layout,with_src", WIDE_CASES)
def test_wide_tiles(E, H, I, T, topk, layout, with_src, monkeypatch):
    """The 256-row-tile large-M K loop (MOE_W4A16_WIDE=1, read at prepare)
    against the oracle, every epilogue."""
    monkeypatch.setenv("MOE_W4A16_WIDE", "1")
    test_multi_block_experts(E, H, I, T, topk, layout, with_src)


@pytest.mark.parametrize("E,H,I,T,topk,layout,with_src", MULTI_BLOCK_CASES)
def test_multi_block_experts(E, H, I, T, topk, layout, with_src):
    """Large-M K-loop GEMMs on experts spanning many 128-row blocks, every
    epilogue (SwiGLU, weighted rows, row-wise BF16 store)."""
    require_gpu()
    import torch
    log(f"case multi-block {layout} E={E} H={H} I={I} T={T} topk={topk} row_src={with_src}")
    w = tiny_weights(E, H, I, seed=E * 11 + T)
    x = synth.activations(91, T, H)
    ids, tw = synth.zipf_routing(92, T, E, topk)
    if layout == "indexed":
        h = prepare(w, "indexed")
        assert "schedule=large-M block=128" in describe(h, T, topk)
        ids_d = i32_dev(ids)
        routing = h.align(ids_d)
        ws = torch.empty(h.workspace_bytes(T, topk, T), dtype=torch.uint8, device="cuda")
        out = h.indexed(bf16_dev(x), ids_d, f32_dev(tw), routing=routing, ws=ws)
        torch.cuda.synchronize()
        ref, inter = O.moe_indexed(x, ids, tw, w, E=E, keep=True)
        check_tol(O.bf16_to_f64(bits_host(out)), ref, "indexed multi-block")
        lay = h.routing_layout(T, topk)
        r = routing.cpu().numpy()
        sid = r[lay.off_sorted:lay.off_sorted + lay.cap]
        a_ws = ws[: lay.cap * I * 2].view(torch.int16).view(lay.cap, I).cpu().numpy().view(np.uint16)
        slots = np.flatnonzero(sid < T * topk)
        ref_a = np.stack([inter["a"][int(f)] for f in sid[slots]])
        frac, mx, within = a_mismatch(a_ws[slots], ref_a, "indexed multi-block")
        assert within and frac < 1e-3
        return
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128, rows=a.shape[0] + 128)
    a_nan = a.copy()
    a_nan[m_idx < 0] = 0x7FC0
    h = prepare(w, "contiguous")
    describe(h, a.shape[0])
    if with_src:
        out = h.contiguous(bf16_dev(a_nan), i32_dev(m_idx), i32_dev(row_src), f32_dev(tw), T, topk)
        ref = O.moe_contiguous(a, m_idx, w, row_src=row_src, topk_w=tw, T=T, topk=topk)
        check_tol(O.bf16_to_f64(bits_host(out)), ref, "contiguous multi-block + combine")
    else:
        out = h.contiguous(bf16_dev(a_nan), i32_dev(m_idx))
        ref = O.moe_contiguous(a, m_idx, w)
        valid = m_idx >= 0
        check_tol(O.bf16_to_f64(bits_host(out))[valid], ref[valid], "contiguous multi-block rows")
