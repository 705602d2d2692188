"""Full-size parity: the workloads at their real shapes, run on the GPU
exactly as the benchmark runs them, checked against the CPU oracle.

Every expert that holds rows is compared at least once:
  * indexed layouts (decode, TP8 shard, EP8 decode share): tokens are chosen
    greedily until every routed expert appears among their top-k rows, and
    those tokens' whole combined outputs are compared;
  * masked: the first and the last valid row of every expert;
  * contiguous prefill: the same greedy cover plus the last tokens routed to
    the three most popular Zipf experts (their rows sit in those experts' last
    128-row block), compared per token against the oracle's indexed result for
    the same routing (the layout-equality pin shows it is the same quantity);
  * EP8 prefill share (48 experts x 512 aligned rows): rows of every expert,
    its last row included.
The oracle's per-expert work (exact dequantisation, the two GEMMs in float64)
is shared by the workloads that use the same weights and runs on a thread
pool; this file only decides which rows to compute and where they go.
"""
import concurrent.futures as cf
import gc
import time

import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import (bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare,
                            require_gpu, weights_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

ORACLE_THREADS = 16


def cover_tokens(ids, first=()):
    """Tokens (ascending) such that every id >= 0 in ``ids`` [T, k] occurs in
    one of their rows: ``first`` plus, greedily, the token adding the most
    experts not yet covered."""
    sets = [set(int(v) for v in r if v >= 0) for r in ids]
    want = set().union(*sets)
    chosen = list(dict.fromkeys(int(t) for t in first))
    seen = set().union(*(sets[t] for t in chosen)) if chosen else set()
    while seen != want:
        t = max(range(len(sets)), key=lambda i: len(sets[i] - seen))
        chosen.append(t)
        seen |= sets[t]
    return np.array(sorted(chosen))


class RowRequests:
    """Rows to run through the oracle, grouped by expert. add() returns a
    handle; result(handle) gives the oracle's float64 y rows after run()."""

    def __init__(self):
        self.rows = {}        # expert -> list of x row arrays
        self.out = {}

    def add(self, e, x_rows):
        lst = self.rows.setdefault(int(e), [])
        start = sum(len(r) for r in lst)
        lst.append(np.asarray(x_rows))
        return int(e), start, len(x_rows)

    def run(self, weights, what):
        """weights: (w13_q, w13_s, w2_q, w2_s) stacked over experts."""
        t0 = time.time()
        experts = sorted(self.rows)

        def one(e):
            x = np.concatenate(self.rows[e])
            w13 = O.dequant(weights[0][e], weights[1][e])
            w2 = O.dequant(weights[2][e], weights[3][e])
            return e, O.expert_ffn(x, w13, w2)[2]
        with cf.ThreadPoolExecutor(ORACLE_THREADS) as ex:
            for i, (e, y) in enumerate(ex.map(one, experts)):
                self.out[e] = y
                if (i + 1) % 96 == 0:
                    log(f"  oracle {what}: {i + 1}/{len(experts)} experts, {time.time() - t0:.0f} s")
        log(f"  oracle {what}: {len(experts)} experts, "
            f"{sum(len(v) for v in self.out.values())} rows in {time.time() - t0:.0f} s")

    def result(self, handle):
        e, start, n = handle
        return self.out[e][start:start + n]


def indexed_request(req, x, ids, tokens):
    """Queue the (token, j) rows of ``tokens``; returns the placement."""
    place = []
    for ti, t in enumerate(tokens):
        for j in range(ids.shape[1]):
            if ids[t, j] >= 0:
                place.append((ti, j, req.add(ids[t, j], x[t:t + 1])))
    return place


def indexed_reference(req, place, tw, tokens, H):
    """The oracle's combine of the queued rows: [len(tokens), H] float64."""
    Y = np.zeros((len(tokens), tw.shape[1], H))
    for ti, j, hd in place:
        Y[ti, j] = req.result(hd)[0]
    return O.combine(Y, tw[tokens])


@pytest.fixture(scope="module")
def kimi():
    """Decode, masked, prefill and the two EP8 shares on the 384-expert
    H=7168 I=2048 weights, run on the GPU; then one oracle pass over every
    expert for all of them."""
    require_gpu()
    import torch
    wl = synth.WORKLOADS[1]
    log("generating 384-expert H=7168 I=2048 weights")
    w = synth.stacked_weights(wl)
    dw = weights_dev(*w)
    torch.cuda.synchronize()
    req = RowRequests()
    res = {}

    # decode, indexed
    log(f"case {wl.name}")
    h = prepare(None, "indexed", dev_weights=dw)
    x = synth.activations(wl.iseed, wl.T, wl.H)
    ids, tw = synth.routing(wl)
    out = O.bf16_to_f64(bits_host(h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))))
    torch.cuda.synchronize()
    tok = cover_tokens(ids)
    res["decode"] = dict(out=out, tok=tok, tw=tw, place=indexed_request(req, x, ids, tok))
    del h

    # masked
    wlm = synth.WORKLOADS[3]
    log(f"case {wlm.name}")
    h = prepare(None, "masked", dev_weights=dw)
    a3, mm = synth.masked_inputs(wlm)
    outm = h.masked(bf16_dev(a3), i32_dev(mm), wlm.expected_m)
    torch.cuda.synchronize()
    rows, place = [], []
    for e in range(wlm.E):
        m = int(mm[e])
        for r in sorted({0, m - 1}) if m > 0 else ():
            rows.append(e * wlm.max_m + r)
            place.append(req.add(e, a3[e, r:r + 1]))
    got = O.bf16_to_f64(bits_host(outm[torch.from_numpy(np.array(rows)).cuda()]))
    res["masked"] = dict(got=got, place=place, experts=int(np.count_nonzero(mm)))
    del h, outm

    # prefill, contiguous with the per-token combine
    wlp = synth.WORKLOADS[2]
    log(f"case {wlp.name}")
    h = prepare(None, "contiguous", dev_weights=dw)
    xp = synth.activations(wlp.iseed, wlp.T, wlp.H)
    idp, twp = synth.routing(wlp)
    a, m_idx, row_src = O.contiguous_layout(xp, idp, wlp.E, 128)
    log(f"  M_pad={a.shape[0]} (valid rows {int((m_idx >= 0).sum())})")
    outp = O.bf16_to_f64(bits_host(h.contiguous(bf16_dev(a), i32_dev(m_idx), i32_dev(row_src),
                                                f32_dev(twp), wlp.T, wlp.topk)))
    torch.cuda.synchronize()
    counts = np.bincount(idp.reshape(-1), minlength=wlp.E)
    hot = np.argsort(-counts, kind="stable")[:3]
    last = [t for e in hot for t in np.flatnonzero(np.any(idp == e, axis=1))[-4:]]
    tokp = cover_tokens(idp, first=[0, wlp.T - 1, *last])
    log(f"  hottest experts {hot.tolist()} with {counts[hot].tolist()} rows; {len(tokp)} tokens")
    res["prefill"] = dict(out=outp, tok=tokp, tw=twp, place=indexed_request(req, xp, idp, tokp),
                          hot_tokens=last)
    del h, a

    # EP8 decode share: experts 0..47 of the 384, global ids through the map
    wle = synth.WORKLOADS[5]
    Eg = wle.extra["global_experts"]
    log(f"case {wle.name}")
    ws = tuple(v[:wle.E] for v in w)
    h = prepare(ws, "indexed")
    xe = synth.activations(wle.iseed, wle.T, wle.H)
    ide, twe = synth.routing(wle)
    emap = np.full(Eg, -1, dtype=np.int32)
    emap[:wle.E] = np.arange(wle.E)
    ovr = {"global_experts": Eg}
    log(f"  {h.describe(wle.T, wle.topk, ovr=ovr)}")
    routing = h.align_ep(i32_dev(ide), i32_dev(emap), Eg, ovr=ovr)
    oute = O.bf16_to_f64(bits_host(h.indexed(bf16_dev(xe), i32_dev(ide), f32_dev(twe),
                                             routing=routing, ovr=ovr)))
    torch.cuda.synchronize()
    loc = O.ep_local_ids(ide, emap)      # local id == global id for this share
    toke = cover_tokens(loc)
    res["ep_decode"] = dict(out=oute, tok=toke, tw=twe, place=indexed_request(req, xe, loc, toke),
                            none=np.flatnonzero(np.all(loc < 0, axis=1)))
    del h, routing

    # EP8 prefill share: 48 experts x 512 aligned rows, no combine
    wlg = synth.WORKLOADS[6]
    rpe = wlg.extra["rows_per_expert"]
    log(f"case {wlg.name}")
    h = prepare(ws, "contiguous")
    ag = synth.activations(wlg.iseed, wlg.E * rpe, wlg.H)
    mg = np.repeat(np.arange(wlg.E, dtype=np.int32), rpe)
    log(f"  {h.describe(wlg.E * rpe)}")
    outg = h.contiguous(bf16_dev(ag), i32_dev(mg))
    torch.cuda.synchronize()
    rows, place = [], []
    for e in range(wlg.E):
        sel = np.unique(np.r_[e * rpe + np.arange(0, rpe, 97) + e % 7, e * rpe + rpe - 1])
        rows.extend(sel.tolist())
        place.append(req.add(e, ag[sel]))
    got = O.bf16_to_f64(bits_host(outg[torch.from_numpy(np.array(rows)).cuda()]))
    res["ep_prefill"] = dict(got=got, place=place)
    del h, outg

    del dw
    gc.collect()
    torch.cuda.empty_cache()
    req.run(w, "384 experts, H=7168 I=2048")
    yield req, res


def test_full_decode_indexed(kimi):
    req, res = kimi
    r = res["decode"]
    wl = synth.WORKLOADS[1]
    assert np.all(np.isfinite(r["out"]))
    assert np.all(np.abs(r["out"]).sum(axis=1) > 0)
    ref = indexed_reference(req, r["place"], r["tw"], r["tok"], wl.H)
    check_tol(r["out"][r["tok"]], ref, f"{wl.name}: {len(r['tok'])} tokens covering every expert")


def test_full_masked(kimi):
    req, res = kimi
    r = res["masked"]
    ref = np.concatenate([req.result(hd) for hd in r["place"]])
    check_tol(r["got"], ref, f"masked: first and last valid row of all {r['experts']} experts with rows")


def test_full_prefill_contiguous(kimi):
    req, res = kimi
    r = res["prefill"]
    wl = synth.WORKLOADS[2]
    assert np.all(np.isfinite(r["out"]))
    assert len(r["tok"]) >= 64
    ref = indexed_reference(req, r["place"], r["tw"], r["tok"], wl.H)
    check_tol(r["out"][r["tok"]], ref, f"{wl.name}: {len(r['tok'])} tokens covering every expert")
    hot = np.isin(r["tok"], r["hot_tokens"])
    check_tol(r["out"][r["tok"][hot]], ref[hot], "prefill: last tokens of the three hottest experts")


def test_full_ep8_share_decode(kimi):
    req, res = kimi
    r = res["ep_decode"]
    wl = synth.WORKLOADS[5]
    assert np.all(r["out"][r["none"]] == 0)
    ref = indexed_reference(req, r["place"], r["tw"], r["tok"], wl.H)
    check_tol(r["out"][r["tok"]], ref, f"{wl.name}: {len(r['tok'])} tokens covering the 48 experts")


def test_full_ep8_share_prefill_grouped(kimi):
    req, res = kimi
    r = res["ep_prefill"]
    ref = np.concatenate([req.result(hd) for hd in r["place"]])
    check_tol(r["got"], ref, f"EP8 prefill share: {len(ref)} rows over all 48 experts")


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
    del h
    assert np.all(np.isfinite(out))
    tok = cover_tokens(ids, first=[0, wl.T - 1])
    req = RowRequests()
    place = indexed_request(req, x, ids, tok)
    req.run(w, "TP8 shard, 384 experts, I=256")
    ref = indexed_reference(req, place, tw, tok, wl.H)
    check_tol(out[tok], ref, f"{wl.name}: {len(tok)} tokens covering every expert")


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
