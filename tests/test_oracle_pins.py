"""Pins for the CPU oracle (CPU only).

Each test checks the oracle against something other than itself: a library
special case (torch's float32 -> bfloat16 cast, torch float32 matmul),
hand-derived fixtures under tests/golden/, exact rational arithmetic, Python
brute force straight from the definitions, closed forms (one-hot weights) and
invariants (the linear-split identity from the DFlash audit, section 2; layout
equality; pad rows contribute nothing). test_planted_mistakes_are_caught plants
plausible mistakes in the oracle and checks that a pin fails for each.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import moe_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Independent helpers (not the oracle's methods)
# --------------------------------------------------------------------------

def _bf16_val(b: int) -> Fraction:
    if b & 0x7F80 == 0x7F80:
        return Fraction(2) ** 128 * (-1 if b & 0x8000 else 1)  # inf as 2^128 for rounding
    return Fraction(struct.unpack("<f", struct.pack("<I", b << 16))[0])


def bf16_nearest_exact(x: float) -> int:
    """Nearest BF16 to a double by exact rational comparison of the two
    neighbours; ties go to the even mantissa."""
    if math.isnan(x):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    ax = abs(x)
    if ax == 0:
        return sign
    fx = Fraction(ax)
    b = struct.unpack("<I", struct.pack("<f", float(np.float32(min(ax, 3.0e38)))))[0] >> 16
    while b > 0 and _bf16_val(b) > fx:
        b -= 1
    while b < 0x7F80 and _bf16_val(b + 1) <= fx:
        b += 1
    if b >= 0x7F80:
        return sign | 0x7F80
    lo, hi = _bf16_val(b), _bf16_val(b + 1)
    dlo, dhi = fx - lo, hi - fx
    pick = b if (dlo < dhi or (dlo == dhi and b % 2 == 0)) else b + 1
    return sign | pick


def bf16_from_f32_bits_formula(x: float) -> int:
    """Classic float32 bit formula for RNE to BF16 (valid for finite x that
    are exactly representable in float32)."""
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF


def f_bf16(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (b & 0xFFFF) << 16))[0]


def torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# BF16 rounding
# --------------------------------------------------------------------------

def pin_bf16_vs_torch():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    f = u.view(np.float32)
    keep = ~np.isnan(f)
    f = f[keep]
    got = O.bf16_round(f.astype(np.float64))
    ref = torch_bf16_bits(f)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} mismatches, first f32 bits {hex(f[bad[0]].view(np.uint32))}"


def test_bf16_round_matches_torch_on_float32_sweep():
    pin_bf16_vs_torch()


def test_bf16_round_nan_and_inf():
    got = O.bf16_round(np.array([np.nan, np.inf, -np.inf, 1e39, -1e39, 0.0, -0.0]))
    assert got[0] & 0x7F80 == 0x7F80 and got[0] & 0x7F
    assert list(got[1:]) == [0x7F80, 0xFF80, 0x7F80, 0xFF80, 0x0000, 0x8000]


def test_bf16_round_float64_against_exact_rationals():
    """Doubles near BF16 ties, subnormals and the overflow edge, checked with
    exact rational arithmetic (no float32 intermediate)."""
    r = np.random.default_rng(7)
    xs = []
    for b in r.integers(1, 0x7F7F, 400):
        lo, hi = float(_bf16_val(int(b))), float(_bf16_val(int(b) + 1))
        mid = (lo + hi) / 2                     # exact in float64
        xs += [mid, math.nextafter(mid, math.inf), math.nextafter(mid, -math.inf),
               -mid, lo, (lo + mid) / 2]
    xs += [2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126 * 1.5, 1e-45,
           float(_bf16_val(0x7F7F)), float.fromhex("0x1.ff0000001p127"),
           float.fromhex("0x1.ffp127"), 3.0e38, 3.4e38]
    xs += list(r.standard_normal(300) * 10.0 ** r.integers(-30, 30, 300))
    got = O.bf16_round(np.array(xs))
    ref = np.array([bf16_nearest_exact(x) for x in xs], dtype=np.uint16)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


# --------------------------------------------------------------------------
# Unpack and dequant
# --------------------------------------------------------------------------

def _read_rows(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split())
    return rows


def pin_unpack_golden():
    for row in _read_rows("unpack_cases.txt"):
        word = np.array([int(row[0], 16)], dtype=np.uint32).view(np.int32)
        q = O.unpack_nibbles(word.reshape(1, 1))
        assert list(q.reshape(-1)) == [int(v) for v in row[1:]], row


def test_unpack_closed_forms():
    pin_unpack_golden()


def pin_dequant_golden():
    for sb, q, exp in _read_rows("dequant_cases.txt"):
        s_bits, qv, e_bits = int(sb, 16), int(q), int(exp, 16)
        # one word whose nibble 0 is q, padded to one group of 32
        words = np.full((1, 4), 0x88888888, dtype=np.uint32)
        words[0, 0] = 0x88888880 | qv
        w = O.dequant(words.view(np.int32), np.array([[s_bits]], dtype=np.uint16))
        assert int(w[0, 0]) == e_bits, (sb, q, hex(int(w[0, 0])), exp)


def test_dequant_golden():
    pin_dequant_golden()


def pin_dequant_exhaustive():
    """All 16 codes x every non-NaN, finite BF16 scale (65,280 normals plus
    zeros and subnormals) against torch: float32 product (exact: a 4-bit by
    8-bit significand) cast to bfloat16."""
    s_bits = np.arange(1 << 16, dtype=np.uint32)
    s_f32 = (s_bits << 16).view(np.float32)
    ok = np.isfinite(s_f32)
    s_bits, s_f32 = s_bits[ok].astype(np.uint16), s_f32[ok]
    for q in range(16):
        # words with every nibble = q, one group of 32 per scale
        word = np.uint32(int("%X" % q * 8, 16))
        words = np.full((s_bits.size, 4), word, dtype=np.uint32).view(np.int32)
        got = O.dequant(words, s_bits[:, None])[:, 0]
        with np.errstate(over="ignore"):
            prod = np.float32(q - 8) * s_f32
        ref = torch_bf16_bits(prod)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (q, hex(int(s_bits[bad[0]])))


def test_dequant_exhaustive_vs_torch():
    pin_dequant_exhaustive()


def test_dequant_scale_group_indexing():
    """Scale group k//32 along K: each group's scale multiplies exactly its
    32 columns (checked with distinct power-of-two scales per group)."""
    r = np.random.default_rng(3)
    words = r.integers(0, 2**32, (5, 16), dtype=np.uint32).view(np.int32)   # K = 128
    scales = np.array([[0x3F80, 0x4000, 0x3E80, 0x4100]] * 5, dtype=np.uint16)  # 1, 2, .25, 8
    w = O.bf16_to_f64(O.dequant(words, scales))
    q = np.array([[(int(wd) >> (4 * i)) & 0xF for wd in row.view(np.uint32) for i in range(8)]
                  for row in words])
    expect = (q - 8) * np.repeat(np.array([1.0, 2.0, 0.25, 8.0]), 32)[None, :]
    np.testing.assert_array_equal(w, expect)


# --------------------------------------------------------------------------
# Alignment
# --------------------------------------------------------------------------

def _golden_align_cases():
    cases, cur = [], None
    for row in _read_rows("align_cases.txt"):
        if row[0] == "case":
            cur = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in row[1:]}
            cases.append(cur)
        else:
            cur[row[0]] = [int(v) for v in row[1:]]
    return cases


def pin_align_golden():
    for c in _golden_align_cases():
        ids = np.array(c["ids"], dtype=np.int32).reshape(c["T"], c["topk"])
        al = O.align(ids, c["E"], c["block"])
        for key in ("counts", "offsets", "sorted_ids", "block_expert"):
            assert list(al[key]) == c[key], (key, list(al[key]), c[key])
        assert al["total"] == c["total"][0]


def test_align_golden():
    pin_align_golden()


def brute_align(ids, E, B):
    T, k = ids.shape
    pairs = sorted((int(ids[t, j]), t * k + j) for t in range(T) for j in range(k)
                   if 0 <= ids[t, j] < E)
    sorted_ids, block_expert = [], []
    for e in range(E):
        mine = [f for (ee, f) in pairs if ee == e]
        n = -(-len(mine) // B) * B
        sorted_ids += mine + [T * k] * (n - len(mine))
        block_expert += [e] * (n // B)
    cap = T * k + E * (B - 1)
    sorted_ids += [T * k] * (cap - len(sorted_ids))
    block_expert += [-1] * (-(-cap // B) - len(block_expert))
    return sorted_ids, block_expert


def pin_align_bruteforce():
    r = np.random.default_rng(11)
    for (T, k, E, B) in [(1, 1, 1, 1), (7, 2, 5, 4), (33, 8, 16, 16), (50, 3, 40, 128),
                         (64, 8, 384, 16), (5, 4, 3, 1)]:
        ids = r.integers(-1, E + 1, (T, k)).astype(np.int32)    # includes dropped ids
        al = O.align(ids, E, B)
        s, b = brute_align(ids, E, B)
        assert list(al["sorted_ids"]) == s
        assert list(al["block_expert"]) == b


def test_align_bruteforce():
    pin_align_bruteforce()


@pytest.mark.parametrize("seed", [0, 1])
def test_align_invariants(seed):
    w = synth.scaled(synth.WORKLOADS[1], T=96, E=64)
    ids, _ = synth.softmax_routing(seed, w.T, w.E, w.topk)
    for B in (1, 16, 128):
        al = O.align(ids, w.E, B)
        n = ids.size
        assert al["counts"].sum() == n
        assert np.all(al["offsets"] % B == 0)
        valid = al["sorted_ids"][al["sorted_ids"] < n]
        assert sorted(valid.tolist()) == list(range(n))
        assert (al["sorted_ids"] == n).sum() == al["cap"] - n
        # within each expert the order is ascending flat index
        for e in range(w.E):
            seg = al["sorted_ids"][al["offsets"][e]:al["offsets"][e] + al["counts"][e]]
            assert np.all(np.diff(seg) > 0)
            assert np.all(ids.reshape(-1)[seg] == e)


# --------------------------------------------------------------------------
# The layer
# --------------------------------------------------------------------------

def _tiny_problem(E=3, H=64, I=32, T=4, k=2, seed=5):
    r = np.random.default_rng(seed)
    w13_q = r.integers(0, 2**32, (E, 2 * I, H // 8), dtype=np.uint32).view(np.int32)
    w2_q = r.integers(0, 2**32, (E, H, I // 8), dtype=np.uint32).view(np.int32)
    w13_s = torch_bf16_bits((np.abs(r.standard_normal((E, 2 * I, H // 32))) * 0.05 + 1e-3).astype(np.float32))
    w2_s = torch_bf16_bits((np.abs(r.standard_normal((E, H, I // 32))) * 0.05 + 1e-3).astype(np.float32))
    x = torch_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tw = r.random((T, k)).astype(np.float32)
    return x, ids, tw, (w13_q, w13_s, w2_q, w2_s)


def brute_layer(x, ids, tw, weights):
    """Python loops straight from the definitions, float64 sums, exact
    rational BF16 rounding for the intermediate."""
    w13_q, w13_s, w2_q, w2_s = weights
    T, k = ids.shape
    H = x.shape[1]
    I = w13_q.shape[1] // 2

    def wval(wq, ws, e, n, kk):
        word = int(wq[e, n, kk // 8]) & 0xFFFFFFFF
        q = (word >> (4 * (kk % 8))) & 0xF
        return f_bf16(bf16_from_f32_bits_formula((q - 8) * f_bf16(int(ws[e, n, kk // 32]))))

    out = [[0.0] * H for _ in range(T)]
    a_rows = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            xs = [f_bf16(int(v)) for v in x[t]]
            h = [sum(xs[kk] * wval(w13_q, w13_s, e, n, kk) for kk in range(H)) for n in range(2 * I)]
            a = []
            for c in range(I):
                g, u = h[c], h[I + c]
                a.append(f_bf16(bf16_nearest_exact(g / (1.0 + math.exp(-g)) * u)))
            a_rows[t * k + j] = a
            for n in range(H):
                y = sum(a[c] * wval(w2_q, w2_s, e, n, c) for c in range(I))
                out[t][n] += float(tw[t, j]) * y
    return np.array(out), a_rows


def pin_layer_bruteforce():
    x, ids, tw, wts = _tiny_problem()
    ref, a_rows = brute_layer(x, ids, tw, wts)
    got, inter = O.moe_indexed(x, ids, tw, wts, E=3, keep=True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    for f, a in a_rows.items():
        assert [f_bf16(int(b)) for b in inter["a"][f]] == a, f


def test_layer_bruteforce_tiny():
    pin_layer_bruteforce()


def _onehot_weights(E, H, I):
    """q = 9 at k = n mod K and 8 elsewhere, power-of-two scales per expert:
    every dot product has exactly one nonzero term."""
    def mat(N, K, scale_bits):
        q = np.full((N, K), 8, dtype=np.uint32)
        q[np.arange(N), np.arange(N) % K] = 9
        words = np.zeros((N, K // 8), dtype=np.uint32)
        for i in range(8):
            words |= q[:, i::8] << np.uint32(4 * i)
        return words.view(np.int32), np.full((N, K // 32), scale_bits, dtype=np.uint16)
    w13 = [mat(2 * I, H, 0x3F80 - (e << 7)) for e in range(E)]         # 2^-e
    w2 = [mat(H, I, 0x3F00 + (e << 7)) for e in range(E)]              # 2^(e-1)
    return (np.stack([a for a, _ in w13]), np.stack([b for _, b in w13]),
            np.stack([a for a, _ in w2]), np.stack([b for _, b in w2]))


def pin_layer_onehot():
    E, H, I, T, k = 4, 64, 32, 5, 2
    wts = _onehot_weights(E, H, I)
    r = np.random.default_rng(2)
    x = torch_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tw = r.random((T, k)).astype(np.float32)
    got = O.moe_indexed(x, ids, tw, wts, E=E)
    xv = np.vectorize(f_bf16)(x.astype(np.int64))
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            s1, s2 = 2.0 ** -e, 2.0 ** (e - 1)
            a = []
            for c in range(I):
                g, u = s1 * xv[t, c % H], s1 * xv[t, (I + c) % H]
                a.append(f_bf16(bf16_nearest_exact(g / (1.0 + math.exp(-g)) * u)))
            for n in range(H):
                ref[t, n] += float(tw[t, j]) * s2 * a[n % I]
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=0)


def test_layer_onehot_exact():
    pin_layer_onehot()


def pin_unfused_onehot():
    """The unfused steps on one-hot weights: every output of gate_up_rows and
    down_rows is one BF16 input times a power of two (exact), and
    swiglu_rows equals z * expit(z) * u (scipy's logistic function) rounded
    once to BF16 by the exact-rational rounder above."""
    from scipy.special import expit
    E, H, I, T = 2, 64, 32, 6
    w13_q, w13_s, w2_q, w2_s = _onehot_weights(E, H, I)
    r = np.random.default_rng(5)
    x = torch_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    xv = np.vectorize(f_bf16)(x.astype(np.int64))
    for e in range(E):
        s1, s2 = 2.0 ** -e, 2.0 ** (e - 1)
        h = O.gate_up_rows(x, O.dequant(w13_q[e], w13_s[e]))
        hv = np.vectorize(f_bf16)(h.astype(np.int64))
        assert np.array_equal(hv, s1 * xv[:, np.arange(2 * I) % H])
        a = O.swiglu_rows(h)
        g, u = hv[:, :I], hv[:, I:]
        ref_a = np.vectorize(lambda v: bf16_nearest_exact(v))(g * expit(g) * u)
        assert np.array_equal(np.vectorize(f_bf16)(a.astype(np.int64)),
                              np.vectorize(f_bf16)(ref_a.astype(np.int64)))
        y = O.down_rows(a, O.dequant(w2_q[e], w2_s[e]))
        av = np.vectorize(f_bf16)(a.astype(np.int64))
        assert np.array_equal(np.vectorize(f_bf16)(y.astype(np.int64)), s2 * av[:, np.arange(H) % I])
    # closed forms: silu(0) = 0, a zero up half gives 0, silu(30) = 30 to within 2^-40
    h = torch_bf16_bits(np.array([[0.0, 30.0, 1.5, 0.0]], dtype=np.float32))
    a = np.vectorize(f_bf16)(O.swiglu_rows(h).astype(np.int64))
    assert a[0, 0] == 0.0 and a[0, 1] == 0.0
    h = torch_bf16_bits(np.array([[30.0, 2.0]], dtype=np.float32))
    assert f_bf16(int(O.swiglu_rows(h)[0, 0])) == 60.0


def test_unfused_steps_onehot():
    pin_unfused_onehot()


def pin_unfused_bruteforce():
    """gate_up_rows / down_rows on tiny random inputs against exact rational
    dot products rounded to the nearest BF16 by exact comparison."""
    r = np.random.default_rng(9)
    H, I, T = 32, 16, 3
    words = r.integers(0, 2 ** 32, size=(2 * I, H // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    scales = torch_bf16_bits((np.abs(r.standard_normal((2 * I, H // 32))) * 0.05 + 1e-3).astype(np.float32))
    w = O.dequant(words, scales)
    x = torch_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    got = O.gate_up_rows(x, w)
    wv = [[_bf16_val(int(b)) for b in row] for row in w]
    for t in range(T):
        xv = [_bf16_val(int(b)) for b in x[t]]
        for n in range(2 * I):
            exact = sum((xv[k] * wv[n][k] for k in range(H)), Fraction(0))
            assert int(got[t, n]) == bf16_nearest_exact(exact), (t, n)
    a = O.swiglu_rows(got)
    w2 = w[:, :I]                            # any BF16 matrix [H', I] serves as W2
    y = O.down_rows(a, w2)
    w2v = [[_bf16_val(int(b)) for b in row] for row in w2]
    for t in range(T):
        av = [_bf16_val(int(b)) for b in a[t]]
        for n in range(w2.shape[0]):
            exact = sum((av[k] * w2v[n][k] for k in range(I)), Fraction(0))
            assert int(y[t, n]) == bf16_nearest_exact(exact), (t, n)


def test_unfused_steps_bruteforce():
    pin_unfused_bruteforce()


def pin_ep_shards():
    """Expert parallelism: the global id -> local id map agrees with a
    brute-force loop, and the layer outputs of disjoint shards (contiguous
    and round-robin placements of 8 experts over 4 GPUs) sum to the
    unsharded layer (float64; only the order of additions differs)."""
    x, ids, tw, (w13_q, w13_s, w2_q, w2_s) = _tiny_problem(H=64, I=32, E=8, T=9, k=3)
    ids = ids.copy()
    ids[2, 1] = -1
    ids[5, 0] = 11                                # outside the global pool
    full = O.moe_indexed(x, ids, tw, (w13_q, w13_s, w2_q, w2_s), E=8)
    for place in ([0, 0, 1, 1, 2, 2, 3, 3], [0, 1, 2, 3, 0, 1, 2, 3]):
        total = np.zeros_like(full)
        for g in range(4):
            mine = [e for e in range(8) if place[e] == g]
            emap = np.full(8, -1, dtype=np.int32)
            emap[mine] = np.arange(len(mine))
            loc = O.ep_local_ids(ids, emap)
            for t in range(ids.shape[0]):
                for j in range(ids.shape[1]):
                    gid = int(ids[t, j])
                    want = int(emap[gid]) if 0 <= gid < 8 else -1
                    assert int(loc[t, j]) == want
            sub = tuple(a[mine] for a in (w13_q, w13_s, w2_q, w2_s))
            total += O.moe_indexed(x, loc, tw, sub, E=len(mine))
        np.testing.assert_allclose(total, full, rtol=1e-12, atol=1e-12 * np.abs(full).max())


def test_ep_shards_sum_to_the_layer():
    pin_ep_shards()


def pin_split_identity():
    """concat(h_i) . W^T = sum_i h_i . W_i^T with K split at multiples of 32
    (DFlash audit, section 2). Dequantising a K-slice of the packed words and
    its scale columns must give the same BF16 weights as slicing the full
    dequantisation, and the segment products must sum to the full product."""
    x, ids, tw, (w13_q, w13_s, w2_q, w2_s) = _tiny_problem(H=128, I=64)
    full = O.dequant(w13_q[0], w13_s[0])
    xf = O.bf16_to_f64(x)
    whole = xf @ O.bf16_to_f64(full).T
    acc = np.zeros_like(whole)
    for a, b in [(0, 32), (32, 96), (96, 128)]:
        part = O.dequant(w13_q[0][:, a // 8:b // 8], w13_s[0][:, a // 32:b // 32])
        assert np.array_equal(part, full[:, a:b])
        acc += xf[:, a:b] @ O.bf16_to_f64(part).T
    np.testing.assert_allclose(acc, whole, rtol=1e-12, atol=1e-12 * np.abs(whole).max())


def test_split_identity():
    pin_split_identity()


def pin_layout_equality():
    """The same routing as indexed, contiguous and masked gives identical y
    per routed row."""
    E, H, I, T, k = 6, 64, 32, 9, 3
    x, ids, tw, wts = _tiny_problem(E=E, H=H, I=I, T=T, k=k, seed=9)
    _, inter = O.moe_indexed(x, ids, tw, wts, E=E, keep=True)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, block=128)
    y_c = O.moe_contiguous(a, m_idx, wts)
    out_c = O.moe_contiguous(a, m_idx, wts, row_src=row_src, topk_w=tw, T=T, topk=k)
    out_i = O.moe_indexed(x, ids, tw, wts, E=E)
    assert np.array_equal(out_c, out_i)
    for r in np.flatnonzero(row_src >= 0):
        assert np.array_equal(y_c[r], inter["y"][int(row_src[r])])
    max_m = 8
    a3 = np.zeros((E, max_m, H), dtype=np.uint16)
    masked_m = np.zeros(E, dtype=np.int32)
    where = {}
    for f in range(T * k):
        e = int(ids.reshape(-1)[f])
        a3[e, masked_m[e]] = x[f // k]
        where[f] = e * max_m + masked_m[e]
        masked_m[e] += 1
    y_m = O.moe_masked(a3, masked_m, wts)
    for f, row in where.items():
        assert np.array_equal(y_m[row], inter["y"][f])


def test_layout_equality():
    pin_layout_equality()


def test_pad_rows_do_not_leak():
    """NaN in contiguous pad rows, in masked rows beyond masked_m and in
    unrouted tokens leaves every valid output bit-identical."""
    E, H, I, T, k = 5, 64, 32, 8, 2
    x, ids, tw, wts = _tiny_problem(E=E, H=H, I=I, T=T, k=k, seed=4)
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, block=128)
    base = O.moe_contiguous(a, m_idx, wts, row_src=row_src, topk_w=tw, T=T, topk=k)
    a_nan = a.copy()
    a_nan[m_idx < 0] = 0x7FC0
    assert np.array_equal(O.moe_contiguous(a_nan, m_idx, wts, row_src=row_src, topk_w=tw, T=T, topk=k), base)
    a3 = np.asarray(synth.activations(1, E * 6, H)).reshape(E, 6, H)
    mm = np.array([0, 6, 3, 1, 2], dtype=np.int32)
    y = O.moe_masked(a3, mm, wts)
    a3n = a3.copy()
    for e in range(E):
        a3n[e, mm[e]:] = 0x7FC0
    y2 = O.moe_masked(a3n, mm, wts)
    valid = np.concatenate([np.arange(e * 6, e * 6 + mm[e]) for e in range(E)])
    assert np.array_equal(y[valid], y2[valid])
    assert np.all(np.isnan(y2[np.setdiff1d(np.arange(E * 6), valid)]))
    # dropped ids (-1) route nowhere: a NaN token that is only "routed" to -1
    ids2 = ids.copy()
    ids2[0, :] = -1
    x2 = x.copy()
    x2[0] = 0x7FC0
    out = O.moe_indexed(x2, ids2, tw, wts, E=E)
    assert np.all(out[0] == 0) and np.all(np.isfinite(out))


def test_expert_matmul_vs_torch_fp32():
    x, ids, tw, (w13_q, w13_s, w2_q, w2_s) = _tiny_problem(H=256, I=128, T=16)
    h, a, y = O.expert_ffn(x, O.dequant(w13_q[1], w13_s[1]), O.dequant(w2_q[1], w2_s[1]))
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    w13t = torch.from_numpy(O.dequant(w13_q[1], w13_s[1]).view(np.int16)).view(torch.bfloat16).float()
    ht = (xt @ w13t.T).double().numpy()
    np.testing.assert_allclose(h, ht, rtol=1e-5, atol=1e-5 * np.abs(ht).max())
    w2t = torch.from_numpy(O.dequant(w2_q[1], w2_s[1]).view(np.int16)).view(torch.bfloat16).float()
    at = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float()
    yt = (at @ w2t.T).double().numpy()
    np.testing.assert_allclose(y, yt, rtol=1e-5, atol=1e-5 * np.abs(yt).max())


def test_compare_metrics():
    ref = np.array([3.0, -4.0])
    m = O.compare(ref * (1 + 1e-3), ref)
    assert abs(m["rel_fro"] - 1e-3) < 1e-12
    assert abs(m["rms"] - math.sqrt(12.5)) < 1e-12


def pin_compare_golden():
    """The comparison's four figures on hand-worked 4-element cases
    (tests/golden/compare_cases.txt derives each one)."""
    for row in _read_rows("compare_cases.txt"):
        ref = np.array([float.fromhex(v) for v in row[1:5]])
        got = np.array([float.fromhex(v) for v in row[5:9]])
        rms, rel, mx, floor = (float(v) for v in row[9:13])
        m = O.compare(got, ref)
        for key, want in (("rms", rms), ("rel_fro", rel), ("max_abs_over_rms", mx), ("bf16_floor", floor)):
            assert abs(m[key] - want) <= 1e-15 + 1e-13 * abs(want), (row[0], key, m[key], want)
        assert m["n"] == 4


def test_compare_golden():
    pin_compare_golden()


def pin_permute_golden():
    """Gather into the aligned order, sentinel slots zero
    (tests/golden/permute_cases.txt derives the rows by hand)."""
    rows = _read_rows("permute_cases.txt")
    T, H, k, E, B = (int(v) for v in rows[0])
    x = np.array([[int(v, 16) for v in r] for r in rows[1:1 + T]], dtype=np.uint16)
    ids = np.array([[int(v) for v in r] for r in rows[1 + T:1 + 2 * T]], dtype=np.int32)
    want = np.array([[int(v, 16) for v in r] for r in rows[1 + 2 * T:]], dtype=np.uint16)
    al = O.align(ids, E, B)
    assert al["cap"] == want.shape[0]
    got = O.permute(x, al, k)
    assert got.dtype == np.uint16 and np.array_equal(got, want), got


def test_permute_golden():
    pin_permute_golden()


# --------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail
# --------------------------------------------------------------------------

def _high_first_unpack(words):
    u = np.asarray(words).view(np.uint32)
    shifts = (7 - np.arange(8, dtype=np.uint32)) * 4
    return ((u[..., :, None] >> shifts) & 0xF).reshape(*u.shape[:-1], u.shape[-1] * 8).astype(np.uint8)


def _dequant_zp7(words, s):
    q = O.unpack_nibbles(words).astype(np.float64) - 7.0
    return O.bf16_round(q * np.repeat(O.bf16_to_f64(s), 32, axis=-1))


def _dequant_group8(words, s):
    q = O.unpack_nibbles(words).astype(np.float64) - 8.0
    sf = O.bf16_to_f64(s)
    idx = np.minimum(np.arange(q.shape[-1]) // 8, sf.shape[-1] - 1)
    return O.bf16_round(q * sf[..., idx])


def _ffn_swapped(x, w13, w2):
    x = O.bf16_to_f64(x)
    w = O.bf16_to_f64(w13)
    I = w.shape[0] // 2
    h = x @ w.T
    a = O.bf16_round(O.silu(h[:, I:]) * h[:, :I])
    return h, a, O.bf16_to_f64(a) @ O.bf16_to_f64(w2).T


def _ffn_round_h(x, w13, w2):
    x = O.bf16_to_f64(x)
    w = O.bf16_to_f64(w13)
    I = w.shape[0] // 2
    h = O.bf16_to_f64(O.bf16_round(x @ w.T))
    a = O.bf16_round(O.silu(h[:, :I]) * h[:, I:])
    return h, a, O.bf16_to_f64(a) @ O.bf16_to_f64(w2).T


def _align_unstable(topk_ids, E, block):
    al = ALIGN_ORIG(topk_ids, E, block)
    s = al["sorted_ids"].copy()
    for e in range(E):
        a, c = al["offsets"][e], al["counts"][e]
        s[a:a + c] = s[a:a + c][::-1]
    al["sorted_ids"] = s
    return al


def _round_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(np.abs(x))
    sp = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    r = np.floor(np.abs(x) / sp + 0.5) * sp
    r = np.copysign(np.where(r > O.BF16_MAX, np.inf, r), x)
    out = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


def _swiglu_swapped(h_bits):
    h = O.bf16_to_f64(h_bits)
    I = h.shape[-1] // 2
    return O.bf16_round(O.silu(h[..., I:]) * h[..., :I])


def _gate_up_truncated(x_rows_bits, w13_bits):
    v = O.bf16_to_f64(x_rows_bits) @ O.bf16_to_f64(w13_bits).T
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _compare_floor_doubled(got, ref):
    m = COMPARE_ORIG(got, ref)
    m["bf16_floor"] *= 2
    return m


def _compare_max_abs_halved(got, ref):
    m = COMPARE_ORIG(got, ref)
    m["max_abs_over_rms"] *= 0.5
    return m


def _compare_rel_fro_over_got(got, ref):
    m = COMPARE_ORIG(got, ref)
    g, r = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    m["rel_fro"] = float(np.linalg.norm(g - r) / np.linalg.norm(g))
    return m


def _compare_floor_truncated(got, ref):
    m = COMPARE_ORIG(got, ref)
    r = np.asarray(ref, dtype=np.float64)
    t = ((r.astype(np.float32).view(np.uint32) >> 16) << 16).view(np.float32).astype(np.float64)
    m["bf16_floor"] = float(np.max(np.abs(t - r))) / m["rms"]
    return m


def _compare_floor_over_max(got, ref):
    m = COMPARE_ORIG(got, ref)
    r = np.asarray(ref, dtype=np.float64)
    m["bf16_floor"] = m["bf16_floor"] * m["rms"] / float(np.max(np.abs(r)))
    return m


def _compare_floor_of_got(got, ref):
    m = COMPARE_ORIG(got, ref)
    g = np.asarray(got, dtype=np.float64)
    m["bf16_floor"] = float(np.max(np.abs(O.bf16_to_f64(O.bf16_round(g)) - g))) / m["rms"]
    return m


def _compare_rms_of_sum(got, ref):
    m = COMPARE_ORIG(got, ref)
    r = np.asarray(ref, dtype=np.float64)
    rms2 = float(np.sqrt(np.sum(r * r)))
    m["max_abs_over_rms"] *= m["rms"] / rms2
    m["bf16_floor"] *= m["rms"] / rms2
    m["rms"] = rms2
    return m


def _permute_mod_topk(x_bits, al, topk):
    x = np.asarray(x_bits)
    sid = al["sorted_ids"].astype(np.int64)
    out = np.zeros((sid.size, x.shape[1]), dtype=np.uint16)
    ok = sid < al["sentinel"]
    out[ok] = x[sid[ok] % topk]
    return out


def _permute_pad_last_row(x_bits, al, topk):
    out = PERMUTE_ORIG(x_bits, al, topk)
    sid = al["sorted_ids"]
    out[sid >= al["sentinel"]] = np.asarray(x_bits)[-1]
    return out


def _permute_off_by_one(x_bits, al, topk):
    x = np.asarray(x_bits)
    sid = al["sorted_ids"].astype(np.int64)
    out = np.zeros((sid.size, x.shape[1]), dtype=np.uint16)
    ok = sid < al["sentinel"]
    out[ok] = x[np.minimum((sid[ok] + 1) // topk, x.shape[0] - 1)]
    return out


ALIGN_ORIG = O.align
COMPARE_ORIG = O.compare
PERMUTE_ORIG = O.permute
PINS = [pin_bf16_vs_torch, pin_unpack_golden, pin_dequant_golden, pin_align_golden,
        pin_align_bruteforce, pin_layer_bruteforce, pin_layer_onehot, pin_split_identity,
        pin_layout_equality, pin_unfused_onehot, pin_unfused_bruteforce, pin_ep_shards,
        pin_compare_golden, pin_permute_golden]


@pytest.mark.parametrize("name,attr,bad", [
    ("nibbles high-first", "unpack_nibbles", _high_first_unpack),
    ("zero point 7", "dequant", _dequant_zp7),
    ("scale per 8 along K", "dequant", _dequant_group8),
    ("gate/up swapped", "expert_ffn", _ffn_swapped),
    ("h rounded to bf16", "expert_ffn", _ffn_round_h),
    ("unstable align", "align", _align_unstable),
    ("bf16 ties away from zero", "bf16_round", _round_ties_away),
    ("unfused SwiGLU halves swapped", "swiglu_rows", _swiglu_swapped),
    ("unfused gate_up unrounded h truncated", "gate_up_rows", _gate_up_truncated),
    ("compare: BF16 floor doubled", "compare", _compare_floor_doubled),
    ("compare: max-abs halved", "compare", _compare_max_abs_halved),
    ("compare: rel_fro over ||got||", "compare", _compare_rel_fro_over_got),
    ("compare: floor by truncation", "compare", _compare_floor_truncated),
    ("compare: floor over max|ref|", "compare", _compare_floor_over_max),
    ("compare: floor of got", "compare", _compare_floor_of_got),
    ("compare: rms as sqrt(sum)", "compare", _compare_rms_of_sum),
    ("permute: token = flat % topk", "permute", _permute_mod_topk),
    ("permute: pad slots copy a row", "permute", _permute_pad_last_row),
    ("permute: flat index off by one", "permute", _permute_off_by_one),
])
def test_planted_mistakes_are_caught(monkeypatch, name, attr, bad):
    monkeypatch.setattr(O, attr, bad)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake '{name}' passed every pin"
