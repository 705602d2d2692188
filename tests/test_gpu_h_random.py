"""GPU parity of the layer against the CPU oracle on seeded random shapes:
expert counts from 1 to 40, hidden and intermediate sizes any multiple of 32
(K and N tails of every length), token counts from 1 up, top-k up to 8,
softmax and Zipf routings, every layout, automatic and forced schedules.
Each case is drawn from a fixed seed, so a failure names a reproducible
shape. Tolerance as for every layer output: relFro <= 5e-3, max-abs <=
3e-2 * rms(ref) (or the BF16 output floor + 5e-3 * rms(ref)).
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare, require_gpu
from tests.test_gpu_a_kernels import tiny_weights

pytestmark = pytest.mark.gpu


def _draw_cases(seed=2024, n=28):
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        layout = ["indexed", "indexed", "indexed", "contiguous", "masked"][i % 5]
        E = int(g.integers(1, 41))
        H = 32 * int(g.integers(1, 21))
        I = 32 * int(g.integers(1, 13))
        if g.random() < 0.4:   # whole 128-k chunks: the large-M kernels can take these
            H, I = 128 * max(1, H // 128), 128 * max(1, I // 128)
        T = int(g.integers(1, 261))
        topk = int(g.integers(1, min(E, 8) + 1))
        routing = "zipf" if g.random() < 0.4 else "softmax"
        schedule = int(g.choice([0, 0, 1, 2]))   # 0 automatic, 1 small-M, 2 large-M
        with_src = bool(g.random() < 0.7)
        max_m = int(g.integers(1, 81))
        expected_m = int(g.integers(1, 121))
        cases.append((i, layout, E, H, I, T, topk, routing, schedule, with_src, max_m, expected_m))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("i,layout,E,H,I,T,topk,routing,schedule,with_src,max_m,expected_m", CASES,
                         ids=[f"case{c[0]}-{c[1]}" for c in CASES])
def test_random_shape(i, layout, E, H, I, T, topk, routing, schedule, with_src, max_m, expected_m):
    require_gpu()
    log(f"case random {i}: {layout} E={E} H={H} I={I} T={T} topk={topk} routing={routing} "
        f"schedule={schedule} row_src={with_src} max_m={max_m} expected_m={expected_m}")
    w = tiny_weights(E, H, I, seed=1000 + i)
    if layout == "masked":
        a3 = synth.activations(2000 + i, E * max_m, H).reshape(E, max_m, H)
        mm = synth.rng(3000 + i, 14).integers(0, max_m + 1, size=E).astype(np.int32)
        a3p = a3.copy()
        for e in range(E):
            a3p[e, mm[e]:] = 0x7FC0   # rows past masked_m are NaN: they must not leak
        h = prepare(w, "masked")
        log(f"  {h.describe(max_m, expected_m=expected_m)}")
        out = O.bf16_to_f64(bits_host(h.masked(bf16_dev(a3p), i32_dev(mm), expected_m)))
        ref = O.moe_masked(a3, mm, w)
        valid = np.concatenate([np.arange(e * max_m, e * max_m + mm[e]) for e in range(E)]).astype(np.int64)
        if valid.size:
            check_tol(out[valid], ref[valid], f"random {i} masked")
        return
    x = synth.activations(2000 + i, T, H)
    if routing == "zipf":
        ids, tw = synth.zipf_routing(4000 + i, T, E, topk)
    else:
        ids, tw = synth.softmax_routing(4000 + i, T, E, topk)
    if layout == "indexed":
        ovr = {"schedule": schedule} if schedule else None
        h = prepare(w, "indexed")
        if schedule == 2 and (H % 128 or I % 128):
            # large-M runs whole 128-k chunks: an explicit request is refused
            import w4a16_int4_grouped_amd as M
            with pytest.raises(M.MoeError, match="OVERRIDE_REJECTED"):
                h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw), ovr=ovr)
            return
        log(f"  {h.describe(T, topk, ovr=ovr)}")
        out = h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw), ovr=ovr)
        ref = O.moe_indexed(x, ids, tw, w, E=E)
        check_tol(O.bf16_to_f64(bits_host(out)), ref, f"random {i} indexed")
        return
    a, m_idx, row_src = O.contiguous_layout(x, ids, E, 128)
    a_nan = a.copy()
    a_nan[m_idx < 0] = 0x7FC0   # padding rows are NaN: they must not leak
    h = prepare(w, "contiguous")
    log(f"  {h.describe(a.shape[0])}")
    if with_src:
        out = h.contiguous(bf16_dev(a_nan), i32_dev(m_idx), i32_dev(row_src), f32_dev(tw), T, topk)
        ref = O.moe_contiguous(a, m_idx, w, row_src=row_src, topk_w=tw, T=T, topk=topk)
        check_tol(O.bf16_to_f64(bits_host(out)), ref, f"random {i} contiguous + combine")
    else:
        out = h.contiguous(bf16_dev(a_nan), i32_dev(m_idx))
        ref = O.moe_contiguous(a, m_idx, w)
        valid = m_idx >= 0
        check_tol(O.bf16_to_f64(bits_host(out))[valid], ref[valid], f"random {i} contiguous rows")
