"""The indexed layer without allocation (moe_w4a16_indexed_noalloc): the
same kernels as moe_w4a16_indexed, run on the library's fixed scratch array
instead of a caller's workspace. Its output must equal the allocating entry
point's bit for bit (both are deterministic and share every kernel), call
after call on the shared array: a large-M call, then a smaller small-M call
that finds the first call's contents in the array, then the first again."""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(wl, T, seed):
    w = synth.scaled(wl, T=T, iseed=seed)
    x = synth.activations(w.iseed, T, w.H)
    ids, tw = synth.routing(w)
    return x, ids, tw


def test_noalloc_matches_indexed_call_after_call():
    require_gpu()
    import torch
    import w4a16_int4_grouped_amd as M
    wl = synth.scaled(synth.WORKLOADS[1], E=32, H=1024, I=512, T=0)
    w = synth.stacked_weights(wl)
    h = prepare(w, "indexed")
    cases = [(384, 301), (40, 302), (384, 301)]      # ~96 rows/expert (large-M), then ~10 (small-M)
    for T, seed in cases:
        x, ids, tw = _inputs(wl, T, seed)
        need = h.workspace_bytes(T, wl.topk, T)
        log(f"case noalloc E={wl.E} H={wl.H} I={wl.I} T={T} top-{wl.topk}: {h.describe(T, wl.topk)}, "
            f"workspace {need} of {M.NOALLOC_SCRATCH_BYTES} bytes")
        assert need <= M.NOALLOC_SCRATCH_BYTES
        xd, idd, twd = bf16_dev(x), i32_dev(ids), f32_dev(tw)
        ref = bits_host(h.indexed(xd, idd, twd))
        out = torch.full((T + 1, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        h.indexed_noalloc(xd, idd, twd, out=out[:T])
        torch.cuda.synchronize()
        got = bits_host(out)
        assert np.array_equal(got[:T], ref), f"T={T}: {int(np.sum(got[:T] != ref))} elements differ"
        assert np.all(np.isnan(O.bf16_to_f64(got[T]))), "the call wrote past its output"
        tok = np.array([0, T // 2, T - 1])
        check_tol(O.bf16_to_f64(got[tok]), O.moe_indexed(x, ids, tw, w, E=wl.E, tokens=tok),
                  f"noalloc T={T} tokens {tok.tolist()}")
    del h


def test_noalloc_rejects_a_call_beyond_the_array():
    require_gpu()
    import torch
    import w4a16_int4_grouped_amd as M
    wl = synth.scaled(synth.WORKLOADS[1], E=8, H=2048, I=256, T=0)
    h = prepare(synth.stacked_weights(wl), "indexed")
    T = 4096
    assert h.workspace_bytes(T, wl.topk, T) > M.NOALLOC_SCRATCH_BYTES
    x, ids, tw = _inputs(wl, T, 303)
    out = torch.zeros((T, wl.H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        h.indexed_noalloc(bf16_dev(x), i32_dev(ids), f32_dev(tw), out=out)
    assert ei.value.status == 5
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
    del h
