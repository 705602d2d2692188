"""The seeded input generators: deterministic, independent per stream and
expert (so one expert of a large workload can be regenerated alone for a
sampled oracle check), and shaped as each workload states."""
import numpy as np

import synth


def test_streams_are_deterministic_and_independent():
    a = synth.activations(7, 16, 64)
    assert np.array_equal(a, synth.activations(7, 16, 64))
    assert not np.array_equal(a, synth.activations(8, 16, 64))
    w0, w1 = synth.expert_weights(3, 64, 32, 0), synth.expert_weights(3, 64, 32, 1)
    for p, q in zip(w0, synth.expert_weights(3, 64, 32, 0)):
        assert np.array_equal(p, q)
    assert not np.array_equal(w0[0], w1[0])
    assert not np.array_equal(w0[0][:, :4], w0[2][:4, :4])     # W13 and W2 words come from other streams


def test_one_expert_regenerates_alone():
    wl = synth.scaled(synth.WORKLOADS[1], E=6, H=64, I=32)
    full = synth.stacked_weights(wl)
    part = synth.stacked_weights(wl, experts=[4])
    for a, b, c in zip(full, part, synth.expert_weights(wl.wseed, wl.H, wl.I, 4)):
        assert np.array_equal(a[4], b[4]) and np.array_equal(a[4], c)


def test_weight_draws_cover_the_schema():
    q13, s13, q2, s2 = synth.expert_weights(101, 256, 128, 0)
    assert q13.shape == (256, 32) and s13.shape == (256, 8) and q2.shape == (256, 16) and s2.shape == (256, 4)
    nib = (q13.view(np.uint32)[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    counts = np.bincount(nib.ravel(), minlength=16)
    assert counts.min() > 0.8 * counts.mean()                   # all 16 codes, roughly uniform
    sc = (s13.astype(np.uint32) << 16).view(np.float32)
    assert np.all(sc > 0) and np.all(np.isfinite(sc))           # |N(0,1)| * 0.02 + 1e-3


def test_routings():
    ids, w = synth.softmax_routing(5, 200, 64, 8)
    assert ids.shape == (200, 8) and w.shape == (200, 8)
    assert all(len(set(r)) == 8 for r in ids)                   # distinct experts per token
    assert np.all(np.diff(w, axis=1) <= 0)                      # descending probability
    assert np.all(w.sum(axis=1) < 1.0)                          # chosen softmax mass, not renormalised
    zi, zw = synth.zipf_routing(6, 2000, 64, 8)
    assert all(len(set(r)) == 8 for r in zi)
    pop = np.bincount(zi.ravel(), minlength=64)
    assert pop.max() > 4 * np.median(pop)                       # skewed popularity
    assert np.array_equal(zi, synth.zipf_routing(6, 2000, 64, 8)[0])


def test_workload_shapes():
    for wl in synth.WORKLOADS.values():
        if wl.layout == "masked":
            a3, mm = synth.masked_inputs(synth.scaled(wl, E=8, H=64))
            assert a3.shape == (8, wl.max_m, 64) and mm.min() >= 0 and mm.max() <= wl.max_m
        elif wl.routing != "none":
            small = synth.scaled(wl, T=min(wl.T, 32))
            ids, _ = synth.routing(small)
            E = wl.extra.get("global_experts", wl.E)
            assert ids.shape == (small.T, wl.topk) and ids.min() >= 0 and ids.max() < E
