"""Full-size parity: the workloads at their real shapes, run on the GPU
exactly as the benchmark runs them, checked against the CPU oracle on
sampled tokens / experts (the oracle recomputes those from the same seeded
inputs). The contiguous result is compared with the oracle's indexed result
for the same routing, which the layout-equality pin shows to be the same
quantity."""
import gc

import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import (bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare,
                            require_gpu, weights_dev)

pytestmark = pytest.mark.gpu


def _provider(w):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = (w[0][e], w[1][e], w[2][e], w[3][e])
        return cache[e]
    return get


@pytest.fixture(scope="module")
def kimi():
    require_gpu()
    import torch
    wl = synth.WORKLOADS[1]
    log("generating 384-expert H=7168 I=2048 weights")
    w = synth.stacked_weights(wl)
    dw = weights_dev(*w)
    torch.cuda.synchronize()
    yield wl, w, dw
    del dw
    gc.collect()
    torch.cuda.empty_cache()


def test_full_decode_indexed(kimi):
    import torch
    wl, w, dw = kimi
    log(f"case {wl.name}")
    h = prepare(None, "indexed", dev_weights=dw)
    x = synth.activations(wl.iseed, wl.T, wl.H)
    ids, tw = synth.routing(wl)
    out = bits_host(h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw)))
    torch.cuda.synchronize()
    outf = O.bf16_to_f64(out)
    assert np.all(np.isfinite(outf))
    assert np.all(np.abs(outf).sum(axis=1) > 0)
    sample = np.array([0, wl.T - 1])
    ref = O.moe_indexed(x, ids, tw, _provider(w), E=wl.E, tokens=sample)
    check_tol(outf[sample], ref, f"{wl.name} tokens {sample.tolist()}")
    del h


def test_full_masked(kimi):
    import torch
    _, w, dw = kimi
    wl = synth.WORKLOADS[3]
    log(f"case {wl.name}")
    h = prepare(None, "masked", dev_weights=dw)
    a3, mm = synth.masked_inputs(wl)
    out = h.masked(bf16_dev(a3), i32_dev(mm), wl.expected_m)
    torch.cuda.synchronize()
    experts = [0, int(np.argmax(mm)), 200, wl.E - 1]
    experts = [e for e in dict.fromkeys(experts) if mm[e] > 0]
    prov = _provider(w)
    ref = O.moe_masked(a3[experts], mm[experts], lambda i: prov(experts[i]))
    rows_ref, rows_got = [], []
    for i, e in enumerate(experts):
        rows_ref.append(ref[i * wl.max_m:i * wl.max_m + mm[e]])
        rows_got.append(np.arange(e * wl.max_m, e * wl.max_m + mm[e]))
    got = O.bf16_to_f64(bits_host(out[torch.from_numpy(np.concatenate(rows_got)).cuda()]))
    check_tol(got, np.concatenate(rows_ref), f"{wl.name} experts {experts}")
    del h


def test_full_prefill_contiguous(kimi):
    import torch
    _, w, dw = kimi
    wl = synth.WORKLOADS[2]
    log(f"case {wl.name}")
    h = prepare(None, "contiguous", dev_weights=dw)
    x = synth.activations(wl.iseed, wl.T, wl.H)
    ids, tw = synth.routing(wl)
    a, m_idx, row_src = O.contiguous_layout(x, ids, wl.E, 128)
    log(f"  M_pad={a.shape[0]} (valid rows {int((m_idx >= 0).sum())})")
    out = h.contiguous(bf16_dev(a), i32_dev(m_idx), i32_dev(row_src), f32_dev(tw), wl.T, wl.topk)
    torch.cuda.synchronize()
    outf = O.bf16_to_f64(bits_host(out))
    assert np.all(np.isfinite(outf))
    sample = np.array([0, wl.T - 1])
    ref = O.moe_indexed(x, ids, tw, _provider(w), E=wl.E, tokens=sample)
    check_tol(outf[sample], ref, f"{wl.name} tokens {sample.tolist()}")
    del h


def test_full_ep8_share_decode(kimi):
    """One GPU's EP8 share of the decode workload: experts 0..47 of the 384
    (the same weights), global ids through the share's map."""
    import torch
    _, w, _ = kimi
    wl = synth.WORKLOADS[5]
    Eg = wl.extra["global_experts"]
    log(f"case {wl.name}")
    ws = tuple(a[:wl.E] for a in w)
    h = prepare(ws, "indexed")
    x = synth.activations(wl.iseed, wl.T, wl.H)
    ids, tw = synth.routing(wl)
    emap = np.full(Eg, -1, dtype=np.int32)
    emap[:wl.E] = np.arange(wl.E)
    ovr = {"global_experts": Eg}
    log(f"  {h.describe(wl.T, wl.topk, ovr=ovr)}")
    routing = h.align_ep(i32_dev(ids), i32_dev(emap), Eg, ovr=ovr)
    out = O.bf16_to_f64(bits_host(h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw), routing=routing,
                                            ovr=ovr)))
    torch.cuda.synchronize()
    loc = O.ep_local_ids(ids, emap)
    has = np.flatnonzero(np.any(loc >= 0, axis=1))
    none = np.flatnonzero(np.all(loc < 0, axis=1))
    assert np.all(out[none] == 0)
    sample = np.array([has[0], has[len(has) // 2], has[-1]])
    ref = O.moe_indexed(x, loc, tw, _provider(ws), E=wl.E, tokens=sample)
    check_tol(out[sample], ref, f"{wl.name} tokens {sample.tolist()}")
    del h


def test_full_ep8_share_prefill_grouped(kimi):
    """One GPU's EP8 share at prefill: 48 experts x 512 aligned grouped rows
    (contiguous layout, no combine), checked on sampled experts' rows."""
    import torch
    _, w, _ = kimi
    wl = synth.WORKLOADS[6]
    rpe = wl.extra["rows_per_expert"]
    log(f"case {wl.name}")
    ws = tuple(a[:wl.E] for a in w)
    h = prepare(ws, "contiguous")
    total = wl.E * rpe
    a = synth.activations(wl.iseed, total, wl.H)
    m_idx = np.repeat(np.arange(wl.E, dtype=np.int32), rpe)
    log(f"  {h.describe(total)}")
    out = h.contiguous(bf16_dev(a), i32_dev(m_idx))
    torch.cuda.synchronize()
    prov = _provider(ws)
    for e in (0, wl.E - 1):
        rows = np.arange(e * rpe, e * rpe + rpe)[::37]
        w13 = O.dequant(*prov(e)[:2])
        w2 = O.dequant(*prov(e)[2:])
        _, _, y = O.expert_ffn(a[rows], w13, w2)
        got = O.bf16_to_f64(bits_host(out[torch.from_numpy(rows).cuda()]))
        check_tol(got, y, f"{wl.name} expert {e} rows {rows[:3].tolist()}..")
    del h


def test_full_tp8_shard_indexed():
    require_gpu()
    import torch
    wl = synth.WORKLOADS[4]
    log(f"case {wl.name}")
    w = synth.stacked_weights(wl)
    h = prepare(w, "indexed")
    x = synth.activations(wl.iseed, wl.T, wl.H)
    ids, tw = synth.routing(wl)
    out = O.bf16_to_f64(bits_host(h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out))
    sample = np.array([0, wl.T // 2, wl.T - 1])
    ref = O.moe_indexed(x, ids, tw, _provider(w), E=wl.E, tokens=sample)
    check_tol(out[sample], ref, f"{wl.name} tokens {sample.tolist()}")


def test_full_tiny_config_every_token():
    require_gpu()
    wl = synth.WORKLOADS[0]
    w = synth.stacked_weights(wl)
    h = prepare(w, "indexed")
    x = synth.activations(wl.iseed, wl.T, wl.H)
    ids, tw = synth.routing(wl)
    out = O.bf16_to_f64(bits_host(h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))))
    ref = O.moe_indexed(x, ids, tw, w, E=wl.E)
    check_tol(out, ref, wl.name)
